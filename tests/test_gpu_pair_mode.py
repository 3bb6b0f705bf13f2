"""Decode with one workgroup per (sequence, head) pair: when the pairs are few and the caller's
bound max_ctx is short, pass 1 gives each pair a workgroup whose wavefronts split its tiles and
combine their softmax states in LDS, so the one-shot calls launch no merge. The same inputs with
a loose bound take the equal chunks of the whole work list and the merge. Both against the
oracle over the generated inputs; in each mode the one-shot call equals pass 1 followed by the
merge bit for bit (after pass 1 in pair mode the merge changes nothing)."""
import numpy as np
import pytest

import workloads
from oracle.caches import ContigCache
from tests.gpu_util import TD, TOL, check, dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _paged_setup

pytestmark = pytest.mark.gpu

TIGHT, LOOSE = 512, 4096   # max_ctx: 32 tiles (pair mode for few pairs) / 256 tiles (chunks)


@pytest.mark.parametrize("dtype,D,G", [("f16", 128, 1), ("f32", 64, 1), ("e4m3", 128, 1),
                                       ("i8", 64, 1), ("f16", 128, 8), ("f16", 64, 4),
                                       ("e4m3", 128, 2), ("f32", 128, 3)])
def test_pair_mode_and_chunks_match_oracle(dtype, D, G):
    d = dev()
    lens = [0, 1, 15, 16, 17, 100, 300, 512]
    H = 3
    note(f"pair mode paged {dtype} D={D} G={G}")
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, lens, H=H, seed=11)
    tables, tl = pool.block_table(seqs)
    qdt = "f32" if dtype == "f32" else "f16"
    q = workloads.normal(g, (len(lens), H * G, D), qdt)
    qd, td, tld = to_dev(q, d), to_dev(tables, d), to_dev(tl, d)
    want = ref.decode(q, tables, tl, scale_of(D))
    tol = TOL["f32"] if dtype == "f32" else TOL["f16"]
    for max_ctx in (TIGHT, LOOSE):
        one = kvc.decode_gqa_paged(qd, layer, td, tld, max_ctx, scale=scale_of(D))
        out, ws = kvc.decode_gqa_partial_paged(qd, layer, td, tld, max_ctx, scale=scale_of(D))
        kvc.decode_gqa_merge(len(lens), H, G, D, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int16) if one.dtype == torch.float16 else one,
                           out.view(torch.int16) if out.dtype == torch.float16 else out)
        check(one.float().cpu().numpy(), want, tol, f"max_ctx={max_ctx}")
        assert one[0].float().abs().sum().item() == 0.0   # the empty sequence


def test_pair_mode_window_and_fused_append():
    d = dev()
    note("pair mode: window and fused append")
    D, H, W = 128, 4, 100
    lens = [300, 450, 5, 0]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, lens, H=H, seed=12)
    tables, tl = pool.block_table(seqs)
    q = workloads.normal(g, (len(lens), H, D), "f16")
    qd, td, tld = to_dev(q, d), to_dev(tables, d), to_dev(tl, d)
    want = ref.decode(q, tables, tl, scale_of(D), window=W)
    for max_ctx in (TIGHT, LOOSE):
        got = kvc.decode_window_paged(qd, layer, td, tld, max_ctx, W, scale=scale_of(D))
        torch.cuda.synchronize()
        check(got.float().cpu().numpy(), want, TOL["f16"], f"window max_ctx={max_ctx}")
    # fused append on a contiguous fp32 cache (the tiny char-GPT shape): output and cache equal
    # the separate writer followed by the decode, in both modes
    B, H, D, S = 2, 6, 64, 256
    gen = workloads.rng(13)
    K = workloads.normal(gen, (B, S, H, D), "f32")
    V = workloads.normal(gen, (B, S, H, D), "f32")
    Q = workloads.normal(gen, (B, H, D), "f32")
    L = [200, 33]
    for max_ctx in (S, LOOSE):
        kc = torch.full((B, H, S, D), float("nan"), dtype=torch.float32, device=d)
        vc = torch.full_like(kc, float("nan"))
        ref_c = ContigCache(B, H, S, D, "f32", fill=np.nan)
        for b in range(B):
            pos = np.zeros(B, np.int32)
            kvc.append_contig(kc[b:b + 1], vc[b:b + 1], to_dev(pos[:1], d),
                              to_dev(K[b:b + 1, :L[b] - 1], d), to_dev(V[b:b + 1, :L[b] - 1], d))
        kf, vf = kc.clone(), vc.clone()
        last_k = np.stack([K[b, L[b] - 1] for b in range(B)])
        last_v = np.stack([V[b, L[b] - 1] for b in range(B)])
        kvc.append_contig(kc, vc, to_dev(np.array(L, np.int32) - 1, d),
                          to_dev(last_k[:, None], d), to_dev(last_v[:, None], d))
        lens_d = to_dev(np.array(L, np.int32), d)
        sep = kvc.decode_attn_contig(to_dev(Q, d), kc, vc, lens_d, max_ctx, scale=0.125)
        fused = kvc.append_decode_contig(to_dev(Q, d), kf, vf, lens_d, to_dev(last_k, d),
                                         to_dev(last_v, d), max_ctx, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(fused, sep)
        assert torch.equal(torch.nan_to_num(kf, 7.0), torch.nan_to_num(kc, 7.0))
        assert torch.equal(torch.nan_to_num(vf, 7.0), torch.nan_to_num(vc, 7.0))
        for b in range(B):
            ref_c.K[b, :, :L[b]] = K[b, :L[b]].transpose(1, 0, 2)
            ref_c.V[b, :, :L[b]] = V[b, :L[b]].transpose(1, 0, 2)
        check(fused.cpu().numpy(), ref_c.decode(Q, L, 0.125), TOL["f32"], f"fused max_ctx={max_ctx}")


def test_merge_needed_query_matches_what_pass_1_leaves():
    """kvc_decode_merge_needed against what pass 1 does, for every pass-1 family (multi-head,
    grouped-query on the matrix cores and on the vector kernel, window, fused append; paged and
    contiguous), tight and loose bounds: when the query says no merge, pass 1 alone (out
    poisoned with NaN first) equals the one-shot call bit for bit; when it says a merge is
    needed, pass 1 alone leaves some rows unwritten. The LLaMA-13B and parallel-sampling bench
    shapes are asked too."""
    d = dev()
    note("merge-needed query")
    D, H = 128, 4
    lens = [0, 1, 15, 16, 17, 100, 300, 512]
    B = len(lens)
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, lens, H=H, seed=14)
    layer32 = _paged_setup(d, "f32", D, lens, H=H, seed=14)[4]   # same seed: the same tables
    tables, tl = pool.block_table(seqs)
    td, tld = to_dev(tables, d), to_dev(tl, d)
    cap = tables.shape[1] * 16
    seen = set()

    def run(name, G, window, max_ctx, kv="f16", lay=layer):
        q = to_dev(workloads.normal(g, (B, H * G, D), "f16"), d)
        needed = kvc.decode_merge_needed(True, "f16", kv, B, H, D, cap, max_ctx, G=G,
                                         window=window)
        if window:
            one = kvc.decode_window_paged(q, lay, td, tld, max_ctx, window, scale=scale_of(D))
            part = kvc.decode_window_partial_paged(q, lay, td, tld, max_ctx, window,
                                                   scale=scale_of(D),
                                                   out=torch.full_like(q, float("nan")))[0]
        else:
            one = kvc.decode_gqa_paged(q, lay, td, tld, max_ctx, scale=scale_of(D))
            part = kvc.decode_gqa_partial_paged(q, lay, td, tld, max_ctx, scale=scale_of(D),
                                                out=torch.full_like(q, float("nan")))[0]
        torch.cuda.synchronize()
        if needed:
            assert torch.isnan(part).any(), f"{name} max_ctx={max_ctx}: nothing left to merge"
        else:
            assert torch.equal(part.view(torch.int16), one.view(torch.int16)), \
                f"{name} max_ctx={max_ctx}"
        seen.add((name, needed))

    for max_ctx in (TIGHT, LOOSE):
        run("multi-head", 1, 0, max_ctx)
        run("grouped-query matrix cores", 8, 0, max_ctx)
        run("grouped-query vector (fp32 cache)", 2, 0, max_ctx, kv="f32", lay=layer32)
        run("window", 1, 2000, max_ctx)   # span 512 (tight) or 2015 positions (loose)
    # fused append on a contiguous fp16 cache: pass 1 alone against the one-shot call
    S = 600
    for max_ctx in (TIGHT, LOOSE):
        kc = torch.zeros((B, H, S, D), dtype=torch.float16, device=d)
        q = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
        kn = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
        vn = to_dev(workloads.normal(g, (B, H, D), "f16"), d)
        needed = kvc.decode_merge_needed(False, "f16", "f16", B, H, D, S, max_ctx, append=True)
        one = kvc.append_decode_contig(q, kc, kc.clone(), tld, kn, vn, max_ctx, scale=scale_of(D))
        part = kvc.append_decode_partial_contig(q, kc, kc.clone(), tld, kn, vn, max_ctx,
                                                scale=scale_of(D),
                                                out=torch.full_like(q, float("nan")))[0]
        torch.cuda.synchronize()
        if needed:
            assert torch.isnan(part).any()
        else:
            assert torch.equal(part.view(torch.int16), one.view(torch.int16))
        seen.add(("fused append contiguous", needed))
    # every family was seen in both modes
    assert {n for n, _ in seen} == {n for n, k in seen if k} == {n for n, k in seen if not k}
    # the bench shapes: LLaMA-13B (1280 sequence-heads) merges, parallel sampling (320) does not
    assert kvc.decode_merge_needed(True, "f16", "f16", 32, 40, 128, 2064, 2064, append=True)
    assert not kvc.decode_merge_needed(True, "f16", "f16", 8, 40, 128, 1152, 1152, append=True)
