"""Grouped-query decode (shared K/V heads: MQA / GQA) on the GPU vs the CPU oracle.

Query head hq reads K/V head hq // G. Small ragged cases span several tiles and partial tiles;
G covers one wavefront per group (2, 4, 8), groups split over wavefronts (16 = 2 x 8, 6 = 3 x 2)
and MQA (one K/V head). fp32 caches or fp32 queries take the one-head-per-wavefront kernels.
G = 1 must equal the multi-head entry points bit for bit. Unused cache slots hold NaN.
"""
import numpy as np
import pytest

import workloads
from oracle.caches import ContigCache
from tests.gpu_util import TD, TOL, check, dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _paged_setup

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 250, 513, 0, 64]


@pytest.mark.parametrize("dtype,D,H,G", [
    ("f16", 128, 2, 2), ("f16", 128, 2, 4), ("f16", 128, 2, 8), ("f16", 128, 1, 8),
    ("f16", 64, 2, 4), ("f16", 64, 3, 8), ("f16", 128, 2, 16), ("f16", 128, 2, 6),
    ("e4m3", 128, 2, 4), ("e4m3", 128, 2, 8), ("e4m3", 64, 2, 2),
    ("i8", 128, 2, 8), ("i8", 64, 2, 4),
    ("f32", 128, 2, 4), ("f32", 64, 1, 3)])
def test_paged_gqa_against_oracle(dtype, D, H, G):
    d = dev()
    note(f"gqa paged {dtype} D={D} H_kv={H} G={G}")
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, LENS, H=H, seed=G * 7 + D)
    tables, tl = pool.block_table(seqs)
    qdt = "f32" if dtype == "f32" else "f16"
    q = workloads.normal(g, (len(LENS), H * G, D), qdt)
    got = kvc.decode_gqa_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d), max(LENS),
                               scale=scale_of(D))
    torch.cuda.synchronize()
    want = ref.decode(q, tables, tl, scale_of(D))
    check(got.float().cpu().numpy(), want, TOL["f32"] if dtype == "f32" else TOL["f16"],
          f"G={G}")
    assert got[LENS.index(0)].float().abs().sum().item() == 0.0


@pytest.mark.parametrize("dtype,D,G", [("f16", 128, 4), ("f16", 64, 8), ("f32", 128, 2)])
def test_contig_gqa_against_oracle(dtype, D, G):
    d = dev()
    note(f"gqa contig {dtype} D={D} G={G}")
    H, S = 2, 528
    B = len(LENS)
    gen = workloads.rng(300 + G)
    K = workloads.normal(gen, (B, S, H, D), dtype)
    V = workloads.normal(gen, (B, S, H, D), dtype)
    q = workloads.normal(gen, (B, H * G, D), dtype)
    ref = ContigCache(B, H, S, D, dtype, fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=TD[dtype], device=d)
    vc = torch.full_like(kc, float("nan"))
    for b, L in enumerate(LENS):
        if L:
            p = np.full(B, S, np.int32)
            p[b] = 0
            kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K[:, :L], d), to_dev(V[:, :L], d))
            ref.append(p, K[:, :L], V[:, :L])
    got = kvc.decode_gqa_contig(to_dev(q, d), kc, vc, to_dev(np.array(LENS, np.int32), d),
                                max(LENS), scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref.decode(q, LENS, scale_of(D)), TOL[dtype], f"G={G}")


@pytest.mark.parametrize("dtype", ["f16", "e4m3"])
def test_group_of_one_equals_multi_head_bit_for_bit(dtype):
    d = dev()
    note(f"gqa G=1 vs mha {dtype}")
    D, H = 128, 3
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, LENS, H=H, seed=11)
    tables, tl = pool.block_table(seqs)
    q = to_dev(workloads.normal(g, (len(LENS), H, D), "f16"), d)
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    a = kvc.decode_gqa_paged(q, layer, tdv, tlv, max(LENS))
    b = kvc.decode_attn_paged(q, layer, tdv, tlv, max(LENS))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gqa_two_phase_equals_single_call_and_workspace_reuse():
    d = dev()
    note("gqa two-phase")
    D, H, G = 128, 2, 8
    lens = [300, 7, 1000, 64]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, lens, H=H, seed=12)
    tables, tl = pool.block_table(seqs)
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    q = to_dev(workloads.normal(g, (4, H * G, D), "f16"), d)
    a = kvc.decode_gqa_paged(q, layer, tdv, tlv, 1000)
    ws = kvc.new_gqa_workspace(4, H, G, D, device=d)
    ws.fill_(0x5A)
    # the two passes on a reused workspace equal the one-shot call with the same batch bit for
    # bit (the split of the work list depends on the batch, so a smaller batch is compared with
    # its own one-shot call, and with the full batch's rows within the fp16 tolerance)
    for B in (4, 2, 3):
        one = kvc.decode_gqa_paged(q[:B].contiguous(), layer, tdv[:B].contiguous(),
                                   tlv[:B].contiguous(), 1000)
        out, _ = kvc.decode_gqa_partial_paged(q[:B].contiguous(), layer, tdv[:B].contiguous(),
                                              tlv[:B].contiguous(), 1000, workspace=ws)
        kvc.decode_gqa_merge(B, H, G, D, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, one), B
        check(out.float().cpu().numpy(), a[:B].float().cpu().numpy(), TOL["f16"], f"B={B}")
    # a workspace sized for multi-head decode is too small for G = 8 and is refused
    small = kvc.new_workspace(4, H, D, device=d)
    with pytest.raises(kvc.KvcError):
        kvc.decode_gqa_paged(q, layer, tdv, tlv, 1000, workspace=small)


def test_gqa_full_layer():
    """The grouped-query workload at full size (B=32, 64 query heads over 8 K/V heads, D=128,
    lengths U[64,2048]) for one layer: the separate writer + decode, and the fused call the
    benchmark times (equal bit for bit, output and cache); every (sequence, query head) row
    against the oracle over the generated inputs."""
    from oracle.attention import decode_row
    d = dev()
    w = workloads.GQA8_PAGED
    B, H, D, G = w.batch, w.heads, w.head_dim, w.extra["group"]
    note("gqa full layer")
    lens = workloads.llama13b_lengths(w)
    N = int(sum(workloads.blocks_for(L) for L in lens))
    MB = workloads.blocks_for(int(lens.max()))
    pool = kvc.Pool(N, MB, order=workloads.llama13b_pool_order(N, w.seed))
    seqs = [pool.alloc() for _ in range(B)]
    slots = np.concatenate([pool.append([s], int(L))[0] for s, L in zip(seqs, lens)])
    k = workloads.torch_normal((len(slots), H, D), torch.float16, d, w.seed * 100 + 1)
    v = workloads.torch_normal((len(slots), H, D), torch.float16, d, w.seed * 100 + 2)
    # token rows in sequence order: sequence b's are off_b .. off_b + L_b - 1, the last the new one
    off = np.concatenate([[0], np.cumsum(lens)])
    last = torch.from_numpy(off[1:] - 1).to(d)
    prior = np.concatenate([np.arange(off[b], off[b + 1] - 1) for b in range(B)])
    prior_d = torch.from_numpy(prior).to(d)
    layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d)
    fused_layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d)
    kvc.write_paged(layer, torch.from_numpy(slots).to(d), k, v)
    kvc.write_paged(fused_layer, torch.from_numpy(slots[prior]).to(d), k[prior_d], v[prior_d])
    tables, tl = pool.block_table(seqs)
    q = workloads.torch_normal((B, H * G, D), torch.float16, d, w.seed * 100 + 3)
    td, tld = torch.from_numpy(tables).to(d), torch.from_numpy(tl).to(d)
    out = kvc.decode_gqa_paged(q, layer, td, tld, int(tl.max()), scale=w.scale)
    fused = kvc.append_decode_gqa_paged(q, fused_layer, td, tld, k[last].contiguous(),
                                        v[last].contiguous(), int(tl.max()), scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(fused, out)
    assert torch.equal(fused_layer.k_pool.view(torch.int16), layer.k_pool.view(torch.int16))
    assert torch.equal(fused_layer.v_pool.view(torch.int16), layer.v_pool.view(torch.int16))
    qh, oh = q.float().cpu().numpy(), out.float().cpu().numpy()
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    for b in range(B):
        for hq in range(H * G):
            Kr = kh[off[b]:off[b + 1], hq // G]
            Vr = vh[off[b]:off[b + 1], hq // G]
            check(oh[b, hq], decode_row(qh[b, hq], Kr, Vr, w.scale), TOL["f16"], f"b={b} hq={hq}")
