"""Seeded random configurations of paged decode against the oracle: cache dtype, head dim, K/V
heads, query heads per K/V head, batch, a length mix (empty sequences, block boundaries, short
and long ones) and sometimes a rolling window, each drawn per case. The fixed-shape tests pin
named cases; these reach combinations of chunk cuts, segment boundaries and group splits that
the fixed cases do not."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import TOL, check, dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _paged_setup

pytestmark = pytest.mark.gpu


def _lengths(g, B):
    """Per-sequence lengths from a mixture: empty, 1, a block boundary (16k or 16k + 1), short,
    or long."""
    kind = g.integers(0, 5, size=B)
    lens = np.where(kind == 0, 0, 1)
    lens = np.where(kind == 2, 16 * g.integers(1, 20, size=B) + g.integers(0, 2, size=B), lens)
    lens = np.where(kind == 3, g.integers(2, 64, size=B), lens)
    lens = np.where(kind == 4, g.integers(64, 700, size=B), lens)
    return [int(x) for x in lens]


@pytest.mark.parametrize("seed", range(48))
def test_random_paged_decode(seed):
    d = dev()
    g = np.random.default_rng(5000 + seed)
    dtype = str(g.choice(["f32", "f16", "f16", "e4m3", "i8"]))
    D = int(g.choice([64, 128]))
    H = int(g.integers(1, 7))
    G = int(g.choice([1, 1, 2, 3, 4, 8, 16, 32])) if dtype != "f32" else int(g.choice([1, 2, 3]))
    B = int(g.integers(1, 41))
    lens = _lengths(g, B)
    if max(lens) == 0:
        lens[0] = 1
    window = int(g.integers(1, 300)) if g.random() < 0.25 else 0
    note(f"random paged decode seed={seed}: {dtype} D={D} H={H} G={G} B={B} window={window}")
    gen, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, lens, H=H, seed=seed)
    tables, tl = pool.block_table(seqs)
    qdt = "f32" if dtype == "f32" else "f16"
    q = workloads.normal(gen, (B, H * G, D), qdt)
    qd, td, tld = to_dev(q, d), to_dev(tables, d), to_dev(tl, d)
    want = ref.decode(q, tables, tl, scale_of(D), window=window)
    # a tight bound (one workgroup per pair when the pairs are few and short) and a loose one
    # (equal chunks of the whole work list and the merge: over 20 tiles per wavefront)
    for max_ctx in (max(lens), max(lens) + 4096):
        if window:
            got = kvc.decode_window_paged(qd, layer, td, tld, max_ctx, window, scale=scale_of(D))
        elif G > 1:
            got = kvc.decode_gqa_paged(qd, layer, td, tld, max_ctx, scale=scale_of(D))
        else:
            got = kvc.decode_attn_paged(qd, layer, td, tld, max_ctx, scale=scale_of(D))
        torch.cuda.synchronize()
        check(got.float().cpu().numpy(), want, TOL["f32"] if dtype == "f32" else TOL["f16"],
              f"seed={seed} max_ctx={max_ctx}")
        # when kvc_decode_merge_needed says pass 1 leaves nothing to merge, pass 1 alone (out
        # poisoned first) equals the one-shot output bit for bit
        cap = tables.shape[1] * 16
        if not kvc.decode_merge_needed(True, qdt, dtype, B, H, D, cap, max_ctx, G=G,
                                       window=window):
            poison = torch.full_like(got, float("nan"))
            if window:
                part = kvc.decode_window_partial_paged(qd, layer, td, tld, max_ctx, window,
                                                       scale=scale_of(D), out=poison)[0]
            else:
                part = kvc.decode_gqa_partial_paged(qd, layer, td, tld, max_ctx,
                                                    scale=scale_of(D), out=poison)[0]
            torch.cuda.synchronize()
            bits = torch.int16 if got.dtype == torch.float16 else torch.int32
            assert torch.equal(part.view(bits), got.view(bits)), f"seed={seed} max_ctx={max_ctx}"

        # empty sequences give zero rows
        for b, L in enumerate(lens):
            if L == 0:
                assert got[b].float().abs().sum().item() == 0.0


@pytest.mark.parametrize("seed", range(24))
def test_random_paged_prefill(seed):
    """Chunked prefill over random configurations: K/V heads, group size, head dim, sequence
    lengths and chunk sizes (a chunk of 0 .. L new tokens at the end of each sequence; a whole
    prompt; a single token), fp16 or fp32 output, against the oracle."""
    d = dev()
    g = np.random.default_rng(7000 + seed)
    D = int(g.choice([64, 128]))
    H = int(g.integers(1, 4))
    G = int(g.choice([1, 2, 3, 4, 8]))
    B = int(g.integers(1, 9))
    lens = [int(x) for x in g.integers(1, 400, size=B)]
    chunk = []
    for L in lens:
        kind = g.integers(0, 4)
        chunk.append(0 if kind == 0 else L if kind == 1 else 1 if kind == 2
                     else int(g.integers(1, L + 1)))
    out_dt = str(g.choice(["f16", "f32"]))
    note(f"random prefill seed={seed}: D={D} H={H} G={G} B={B} out={out_dt}")
    gen, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, lens, H=H, seed=seed)
    tables, tl = pool.block_table(seqs)
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    total = int(qs[-1])
    if total == 0:
        chunk[0] = 1
        qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
        total = 1
    q = workloads.normal(gen, (total, H * G, D), "f16")
    o = torch.full((total, H * G, D), float("nan"), dtype=torch.float16 if out_dt == "f16"
                   else torch.float32, device=d)
    got = kvc.prefill_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(qs, d), to_dev(tl, d),
                            scale=scale_of(D), out=o)
    torch.cuda.synchronize()
    want = ref.prefill(q, qs, tables, tl, scale_of(D))
    check(got.float().cpu().numpy(), want, TOL["f16"], f"seed={seed}")


@pytest.mark.parametrize("seed", range(16))
def test_random_contig_fused_decode(seed):
    """Contiguous caches through the fused append-and-attend call (multi-head or grouped): the
    output and cache equal the writer + decode path bit for bit, and the output the oracle's."""
    from oracle.caches import ContigCache
    from tests.gpu_util import TD
    d = dev()
    g = np.random.default_rng(9000 + seed)
    dtype = str(g.choice(["f32", "f16"]))
    D = int(g.choice([64, 128]))
    H = int(g.integers(1, 5))
    G = int(g.choice([1, 1, 2, 4, 8, 16, 32])) if dtype == "f16" else int(g.choice([1, 2]))
    B = int(g.integers(1, 17))
    S = int(g.integers(1, 5)) * 64
    lens = [int(x) for x in g.integers(0, S + 1, size=B)]
    note(f"random contig fused seed={seed}: {dtype} D={D} H={H} G={G} B={B} S={S}")
    K = workloads.normal(g, (B, S, H, D), dtype)
    V = workloads.normal(g, (B, S, H, D), dtype)
    q = workloads.normal(g, (B, H * G, D), dtype)
    ref = ContigCache(B, H, S, D, dtype, fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=TD[dtype], device=d)
    vc = torch.full_like(kc, float("nan"))
    for b, L in enumerate(lens):           # positions [0, L-1) already cached
        if L > 1:
            p = np.full(B, S, np.int32)
            p[b] = 0
            kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K[:, :L - 1], d),
                              to_dev(V[:, :L - 1], d))
            ref.append(p, K[:, :L - 1], V[:, :L - 1])
    pos = np.array([L - 1 if L > 0 else S for L in lens], np.int32)
    k_new = K[np.arange(B), np.maximum(pos, 0) % S]
    v_new = V[np.arange(B), np.maximum(pos, 0) % S]
    ref.append(pos, k_new[:, None], v_new[:, None])
    kc2, vc2 = kc.clone(), vc.clone()
    lens_d = to_dev(np.array(lens, np.int32), d)
    qd, kd, vd = to_dev(q, d), to_dev(k_new, d), to_dev(v_new, d)
    mx = max(max(lens), 1)
    if G > 1:
        fused = kvc.append_decode_gqa_contig(qd, kc, vc, lens_d, kd, vd, mx, scale=scale_of(D))
    else:
        fused = kvc.append_decode_contig(qd, kc, vc, lens_d, kd, vd, mx, scale=scale_of(D))
    kvc.append_contig(kc2, vc2, to_dev(pos, d), kd[:, None].contiguous(), vd[:, None].contiguous())
    plain = (kvc.decode_gqa_contig(qd, kc2, vc2, lens_d, mx, scale=scale_of(D)) if G > 1 else
             kvc.decode_attn_contig(qd, kc2, vc2, lens_d, mx, scale=scale_of(D)))
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    np.testing.assert_array_equal(kc.cpu().numpy(), ref.K)
    np.testing.assert_array_equal(vc.cpu().numpy(), ref.V)
    check(fused.float().cpu().numpy(), ref.decode(q, lens, scale_of(D)),
          TOL[dtype], f"seed={seed}")
