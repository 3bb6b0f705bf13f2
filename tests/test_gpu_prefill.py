"""Chunked prefill on the GPU vs the CPU oracle (full causal recompute per chunk).

Each sequence's chunk is the last n_b of its L_b positions (K/V already written): whole prompts
(n_b = L_b), tails of longer sequences (start_pos > 0), single rows, empty chunks, and lengths
that end inside a block. G covers multi-head, pairs of heads and groups of 4 and 8 query heads
per K/V head. Unused cache slots hold NaN.
"""
import numpy as np
import pytest

import workloads
from oracle.caches import ContigCache
from tests.gpu_util import TD, TOL, check, dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _paged_setup

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 250, 513, 0, 64, 300]
CHUNK = [1, 15, 3, 17, 250, 100, 0, 1, 64]


def _q_start(chunk):
    return np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)


@pytest.mark.parametrize("D,H,G,out", [(128, 2, 1, "f16"), (64, 3, 1, "f32"), (128, 2, 2, "f16"),
                                       (128, 1, 4, "f16"), (64, 2, 8, "f16"), (128, 2, 3, "f32")])
def test_paged_prefill_against_oracle(D, H, G, out):
    d = dev()
    note(f"prefill paged D={D} H_kv={H} G={G} out={out}")
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, LENS, H=H, seed=D + G)
    tables, tl = pool.block_table(seqs)
    qs = _q_start(CHUNK)
    q = workloads.normal(g, (int(qs[-1]), H * G, D), "f16")
    o = torch.full((int(qs[-1]), H * G, D), float("nan"), dtype=TD[out], device=d)
    got = kvc.prefill_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(qs, d), to_dev(tl, d),
                            scale=scale_of(D), out=o)
    torch.cuda.synchronize()
    want = ref.prefill(q, qs, tables, tl, scale_of(D))
    check(got.float().cpu().numpy(), want, TOL["f16"], f"G={G}")


@pytest.mark.parametrize("D,G", [(128, 1), (64, 4)])
def test_contig_prefill_against_oracle(D, G):
    d = dev()
    note(f"prefill contig D={D} G={G}")
    H, S = 2, 528
    B = len(LENS)
    gen = workloads.rng(500 + D + G)
    K = workloads.normal(gen, (B, S, H, D), "f16")
    V = workloads.normal(gen, (B, S, H, D), "f16")
    ref = ContigCache(B, H, S, D, "f16", fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=torch.float16, device=d)
    vc = torch.full_like(kc, float("nan"))
    for b, L in enumerate(LENS):
        if L:
            p = np.full(B, S, np.int32)
            p[b] = 0
            kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K[:, :L], d), to_dev(V[:, :L], d))
            ref.append(p, K[:, :L], V[:, :L])
    qs = _q_start(CHUNK)
    q = workloads.normal(gen, (int(qs[-1]), H * G, D), "f16")
    got = kvc.prefill_contig(to_dev(q, d), kc, vc, to_dev(qs, d),
                             to_dev(np.array(LENS, np.int32), d), scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref.prefill(q, qs, LENS, scale_of(D)), TOL["f16"], f"G={G}")


def test_prefill_last_rows_equal_decode():
    """The last row of each chunk is the decode of that query at the full length: the GPU
    prefill and the GPU decode agree to the fp16 output's rounding."""
    d = dev()
    note("prefill last row vs decode")
    D, H = 128, 2
    lens = [40, 17, 300, 2]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, lens, H=H, seed=3)
    tables, tl = pool.block_table(seqs)
    chunk = [40, 5, 77, 2]
    qs = _q_start(chunk)
    q = workloads.normal(g, (int(qs[-1]), H, D), "f16")
    pf = kvc.prefill_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(qs, d), to_dev(tl, d),
                           out=torch.empty((int(qs[-1]), H, D), dtype=torch.float32, device=d))
    last = q[qs[1:] - 1]
    dec = kvc.decode_attn_paged(to_dev(last, d), layer, to_dev(tables, d), to_dev(tl, d),
                                max(lens), out=torch.empty((4, H, D), dtype=torch.float32,
                                                           device=d))
    torch.cuda.synchronize()
    check(pf[torch.from_numpy(qs[1:] - 1).long().to(d)].cpu().numpy(), dec.cpu().numpy(), 1e-5,
          "last rows")


def test_prefill_argument_errors():
    d = dev()
    note("prefill errors")
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", 64, [20], H=1, seed=1)
    tables, tl = pool.block_table(seqs)
    qs = to_dev(_q_start([4]), d)
    q32 = to_dev(workloads.normal(g, (4, 1, 64), "f32"), d)
    with pytest.raises(kvc.KvcError):
        kvc.prefill_paged(q32, layer, to_dev(tables, d), qs, to_dev(tl, d))
    f32layer = kvc.PagedLayer.empty(4, 1, 64, "f32", device=d)
    q16 = q32.half()
    with pytest.raises(kvc.KvcError):
        kvc.prefill_paged(q16, f32layer, to_dev(tables, d), qs, to_dev(tl, d))


def test_prefill_full_size():
    """LLaMA-7B head shapes (32 x 128, fp16): four 2048-token prompts prefilled whole through a
    shuffled paged pool, the benchmark's launch configuration. Against the oracle over the
    generated inputs: every row of two heads per prompt (full_causal), and in every other
    (prompt, head) the first and last rows, the rows either side of each 128-row tile edge of
    the first 512, and 8 random rows (row r: decode_row over positions 0..r, the definition of a
    causal row)."""
    from oracle.attention import decode_row
    from oracle.attention import full_causal
    d = dev()
    w = workloads.LLAMA7B_PREFILL
    B, H, D, T = w.batch, w.heads, w.head_dim, w.ctx
    note("prefill full size")
    N = B * workloads.blocks_for(T)
    pool = kvc.Pool(N, workloads.blocks_for(T), order=workloads.llama13b_pool_order(N, w.seed))
    seqs = [pool.alloc() for _ in range(B)]
    slots = np.concatenate([pool.append([s], T)[0] for s in seqs])
    layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d)
    k = workloads.torch_normal((B * T, H, D), torch.float16, d, w.seed * 100 + 1)
    v = workloads.torch_normal((B * T, H, D), torch.float16, d, w.seed * 100 + 2)
    q = workloads.torch_normal((B * T, H, D), torch.float16, d, w.seed * 100 + 3)
    kvc.write_paged(layer, torch.from_numpy(slots).to(d), k, v)
    tables, tl = pool.block_table(seqs)
    qs = _q_start([T] * B)
    out = kvc.prefill_paged(q, layer, to_dev(tables, d), to_dev(qs, d), to_dev(tl, d),
                            scale=w.scale)
    torch.cuda.synchronize()
    kh, vh, qh = (t.cpu().numpy() for t in (k, v, q))
    oh = out.float().cpu().numpy()
    gen = np.random.default_rng(2)
    edges = [0, 1, 127, 128, 255, 256, 383, 384, 511, 512, T - 1]
    for b in range(B):
        sl = slice(b * T, (b + 1) * T)
        full = set(int(x) for x in gen.choice(H, size=2, replace=False))
        for h in range(H):
            if h in full:
                want = full_causal(qh[sl, h], kh[sl, h], vh[sl, h], w.scale)
                check(oh[sl][:, h], want, TOL["f16"], f"b={b} h={h} all rows")
                continue
            rows = sorted(set(edges) | set(int(x) for x in gen.choice(T, size=8, replace=False)))
            for r in rows:
                want = decode_row(qh[sl][r, h], kh[sl][:r + 1, h], vh[sl][:r + 1, h], w.scale)
                check(oh[sl][r, h], want, TOL["f16"], f"b={b} h={h} row {r}")
