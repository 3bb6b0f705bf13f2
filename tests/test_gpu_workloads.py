"""HIP path vs the CPU oracle at the full workload sizes (one layer each), in the launch
configuration the benchmark uses. Every oracle input comes from the generated inputs (never
from a cache the library wrote): every (sequence, head) output row of the fp16 workloads is
checked; for the 8-bit long-context caches the oracle's own writer encodes every block of
sampled sequences, which must equal the library's codes and scales bit for bit, and every head
of those sequences is checked. Block tables are compared bit for bit. The tiny char-GPT
workload runs in full in test_gpu_parity.py."""
import numpy as np
import pytest

import workloads
from oracle.attention import decode_row
from oracle.caches import PagedCache
from oracle.codecs import e4m3_decode, fp8_write_token
from oracle.pool import PoolModel
from tests.gpu_util import TOL, check, dev, kvc, note, scale_of, torch

pytestmark = pytest.mark.gpu


def test_llama7b_contiguous_full_layer():
    """B=16, H=32, D=128, fp16, S_max=2048: prefill 2047 positions, append one, attend 2048 --
    with the separate writer and with the fused call the benchmark times (equal bit for bit);
    every (sequence, head) row against the oracle over the generated inputs."""
    d = dev()
    w = workloads.LLAMA7B_CONTIG
    B, H, D, S = w.batch, w.heads, w.head_dim, w.s_max
    note("llama7b contiguous full layer")
    kc = torch.full((B, H, S, D), float("nan"), dtype=torch.float16, device=d)
    vc = torch.full_like(kc, float("nan"))
    kn = workloads.torch_normal((B, S, H, D), torch.float16, d, w.seed * 10 + 1)
    vn = workloads.torch_normal((B, S, H, D), torch.float16, d, w.seed * 10 + 2)
    zeros = torch.zeros(B, dtype=torch.int32, device=d)
    kvc.append_contig(kc, vc, zeros, kn[:, :S - 1].contiguous(), vn[:, :S - 1].contiguous())
    kf, vf = kc.clone(), vc.clone()   # the fused call's cache: positions 0 .. S-2
    kvc.append_contig(kc, vc, torch.full((B,), S - 1, dtype=torch.int32, device=d),
                      kn[:, S - 1:].contiguous(), vn[:, S - 1:].contiguous())
    q = workloads.torch_normal((B, H, D), torch.float16, d, w.seed * 10 + 3)
    lens = torch.full((B,), S, dtype=torch.int32, device=d)
    out = kvc.decode_attn_contig(q, kc, vc, lens, S, scale=w.scale)
    fused = kvc.append_decode_contig(q, kf, vf, lens, kn[:, S - 1].contiguous(),
                                     vn[:, S - 1].contiguous(), S, scale=w.scale)
    torch.cuda.synchronize()
    # the cache holds exactly the appended values (bitwise), in [B, H, S, D] order
    assert torch.equal(kc, kn.permute(0, 2, 1, 3)) and torch.equal(vc, vn.permute(0, 2, 1, 3))
    assert torch.equal(fused, out)
    assert torch.equal(kf, kc) and torch.equal(vf, vc)
    got = out.float().cpu().numpy()
    qh = q.float().cpu().numpy()
    knh, vnh = kn.cpu().numpy(), vn.cpu().numpy()   # fp16 [B, S, H, D]
    for b in range(B):
        for h in range(H):
            want = decode_row(qh[b, h], knh[b, :, h], vnh[b, :, h], w.scale)
            check(got[b, h], want, TOL["f16"], f"b={b} h={h}")


def _llama13b_state(d, w, layer_count=1):
    lens = workloads.llama13b_lengths(w)
    N = int(sum(workloads.blocks_for(L) for L in lens)) + w.batch
    MB = workloads.blocks_for(int(lens.max())) + 1
    order = workloads.llama13b_pool_order(N, w.seed)
    pool = kvc.Pool(N, MB, order=order)
    model = PoolModel(N, 16, MB, order=order)
    seqs = [pool.alloc() for _ in range(w.batch)]
    for _ in seqs:
        model.alloc()
    return lens, N, MB, pool, model, seqs


def test_llama13b_paged_full_layer():
    """B=32, H=40, D=128, fp16, lengths U[64, 2048], shuffled pool: prefill L_b - 1 tokens per
    sequence, one decode step (append, write, attend); tables bit-exact against the pool model,
    every (sequence, head) row against the oracle over the generated inputs."""
    d = dev()
    w = workloads.LLAMA13B_PAGED
    B, H, D = w.batch, w.heads, w.head_dim
    note("llama13b paged full layer")
    lens, N, MB, pool, model, seqs = _llama13b_state(d, w)
    slots = np.concatenate([pool.append([s], int(L) - 1)[0] for s, L in zip(seqs, lens)])
    mslots = sum((model.append([s], int(L) - 1)[0] for s, L in zip(seqs, lens)), [])
    assert slots.tolist() == mslots
    layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d, fill=float("nan"))
    k = workloads.torch_normal((len(slots), H, D), torch.float16, d, 31)
    v = workloads.torch_normal((len(slots), H, D), torch.float16, d, 32)
    kvc.write_paged(layer, torch.from_numpy(slots).to(d), k, v)
    step, src, _ = pool.append(seqs, 1)
    mstep, cow = model.append(seqs, 1)
    assert step.tolist() == mstep and len(src) == 0 and cow == []
    kn = workloads.torch_normal((B, H, D), torch.float16, d, 33)
    vn = workloads.torch_normal((B, H, D), torch.float16, d, 34)
    fused_layer = kvc.PagedLayer(layer.k_pool.clone(), layer.v_pool.clone())  # before the append
    kvc.write_paged(layer, torch.from_numpy(step).to(d), kn, vn)
    tables, tl = pool.block_table(seqs)
    mt, ml = model.block_table(seqs)
    assert tables.tolist() == mt and tl.tolist() == ml == lens.tolist()
    q = workloads.torch_normal((B, H, D), torch.float16, d, 35)
    td, tld = torch.from_numpy(tables).to(d), torch.from_numpy(tl).to(d)
    out = kvc.decode_attn_paged(q, layer, td, tld, int(lens.max()), scale=w.scale)
    # the call the benchmark times: the new token stored by pass 1 itself
    fused = kvc.append_decode_paged(q, fused_layer, td, tld, kn, vn, int(lens.max()),
                                    scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(fused, out)
    assert torch.equal(fused_layer.k_pool.view(torch.int16), layer.k_pool.view(torch.int16))
    assert torch.equal(fused_layer.v_pool.view(torch.int16), layer.v_pool.view(torch.int16))
    got = out.float().cpu().numpy()
    qh = q.float().cpu().numpy()
    # oracle rows from the generated inputs: sequence b's first L_b - 1 tokens are rows
    # off_b .. off_b + L_b - 2 of k/v (appended in sequence order), its last is kn[b]/vn[b]
    off = np.concatenate([[0], np.cumsum(lens - 1)])
    kh, vh = k.cpu().numpy(), v.cpu().numpy()          # fp16 [sum(L_b - 1), H, D]
    knh, vnh = kn.cpu().numpy(), vn.cpu().numpy()      # fp16 [B, H, D]
    for b in range(B):
        L = int(tl[b])
        for h in range(H):
            Kb = np.concatenate([kh[off[b]:off[b] + L - 1, h], knh[b, h][None]])
            Vb = np.concatenate([vh[off[b]:off[b] + L - 1, h], vnh[b, h][None]])
            check(got[b, h], decode_row(qh[b, h], Kb, Vb, w.scale), TOL["f16"], f"b={b} h={h}")
    # the appended token of every sequence is where its slot says, bit for bit
    kp = layer.k_pool.cpu().numpy()
    knh = kn.cpu().numpy()
    for b in range(B):
        blk, o = divmod(int(step[b]), 16)
        np.testing.assert_array_equal(kp[blk, :, o], knh[b])


@pytest.mark.parametrize("prompt,copies", [(1024, 0), (1020, 7)])
def test_parallel_sampling_full(prompt, copies):
    """8 candidates share a prompt (refcount 8), then each appends 128 tokens with attention at
    every step (H=40, D=128, fp16). Pools, tables and sampled steps against the oracle; block
    counts against the pages' 2048-slot figure (and the copy-on-write variant's 135 blocks)."""
    d = dev()
    w = workloads.PARALLEL_SAMPLING
    H, D, G = w.heads, w.head_dim, w.extra["generate"]
    note(f"parallel sampling prompt={prompt}")
    N, MB = 160, 80
    g = workloads.rng(w.seed + prompt)
    pool = kvc.Pool(N, MB)
    model = PoolModel(N, 16, MB)
    layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, "f16", fill=np.nan)
    p = pool.alloc()
    model.alloc()
    slots, _, _ = pool.append([p], prompt)
    model.append([p], prompt)
    k = workloads.normal(g, (prompt, H, D), "f16")
    v = workloads.normal(g, (prompt, H, D), "f16")
    kvc.write_paged(layer, torch.from_numpy(slots).to(d), torch.from_numpy(k).to(d),
                    torch.from_numpy(v).to(d))
    ref.write(slots, k, v)
    seqs = [p] + [pool.fork(p) for _ in range(7)]
    for _ in range(7):
        model.fork(p)
    ws = kvc.new_workspace(8, H, D, device=d)
    n_copies = 0
    for step in range(G):
        slots, src, dst = pool.append(seqs, 1)
        ms, cow = model.append(seqs, 1)
        assert slots.tolist() == ms and list(zip(src.tolist(), dst.tolist())) == cow
        n_copies += len(cow)
        if len(cow):
            kvc.copy_blocks(layer, torch.from_numpy(src).to(d), torch.from_numpy(dst).to(d))
            ref.copy_blocks(cow)
        k = workloads.normal(g, (8, H, D), "f16")
        v = workloads.normal(g, (8, H, D), "f16")
        kvc.write_paged(layer, torch.from_numpy(slots).to(d), torch.from_numpy(k).to(d),
                        torch.from_numpy(v).to(d))
        ref.write(slots, k, v)
        tables, tl = pool.block_table(seqs)
        q = workloads.normal(g, (8, H, D), "f16")
        out = kvc.decode_attn_paged(torch.from_numpy(q).to(d), layer,
                                    torch.from_numpy(tables).to(d), torch.from_numpy(tl).to(d),
                                    prompt + G, scale=scale_of(D), workspace=ws)
        if step in (0, 63, G - 1):
            check(out.float().cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), TOL["f16"],
                  f"step {step}")
    assert n_copies == copies
    st = pool.stats()
    assert st["used"] == (128 if prompt == 1024 else 135)
    if prompt == 1024:
        assert st["used"] * 16 == 2048 and st["tokens"] == 8 * (1024 + 128)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(layer.k_pool.cpu().numpy(), ref.K)
    np.testing.assert_array_equal(layer.v_pool.cpu().numpy(), ref.V)


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_q8_long_context_full_layer(fmt):
    """B=64, H=32, D=128, 8-bit codes (e4m3 or int8) with per-block scales, context 4096:
    prefill 4095 tokens per sequence through the 8-bit writer, append one, attend. For sampled
    sequences the oracle's writer encodes every block from the generated inputs; the library's
    codes and scales must equal them bit for bit. Every head of those sequences is then checked
    against the oracle over the oracle's own codes (2e-3) and over the unquantised inputs
    (3e-2)."""
    from oracle.codecs import i8_decode, i8_write_token
    d = dev()
    w = workloads.LONGCTX_FP8 if fmt == "e4m3" else workloads.LONGCTX_I8
    write_token = fp8_write_token if fmt == "e4m3" else i8_write_token
    decode = e4m3_decode if fmt == "e4m3" else i8_decode
    npdt = np.uint8 if fmt == "e4m3" else np.int8
    B, H, D, T = w.batch, w.heads, w.head_dim, w.ctx
    note(f"{fmt} long context full layer")
    nblk = workloads.blocks_for(T)
    N = B * nblk
    pool = kvc.Pool(N, nblk)
    seqs = [pool.alloc() for _ in range(B)]
    slots = pool.append(seqs, T - 1)[0]
    layer = kvc.PagedLayer.empty(N, H, D, fmt, device=d, fill=float("nan"))
    k = workloads.torch_normal((len(slots), H, D), torch.float16, d, 51)
    v = workloads.torch_normal((len(slots), H, D), torch.float16, d, 52)
    kvc.write_paged(layer, torch.from_numpy(slots).to(d), k, v)
    step = pool.append(seqs, 1)[0]
    kn = workloads.torch_normal((B, H, D), torch.float16, d, 53)
    vn = workloads.torch_normal((B, H, D), torch.float16, d, 54)
    kvc.write_paged(layer, torch.from_numpy(step).to(d), kn, vn)
    tables, tl = pool.block_table(seqs)
    assert (tl == T).all()
    q = workloads.torch_normal((B, H, D), torch.float16, d, 55)
    out = kvc.decode_attn_paged(q, layer, torch.from_numpy(tables).to(d),
                                torch.from_numpy(tl).to(d), T, scale=w.scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    qh = q.float().cpu().numpy()
    rng = np.random.default_rng(2)
    for b in sorted(int(x) for x in rng.choice(B, size=3, replace=False)):
        note(f"{fmt} long context: oracle writer over sequence {b}")
        # the sequence's tokens in position order: prefill rows b*(T-1) .. , then the new one
        rows = slice(b * (T - 1), (b + 1) * (T - 1))
        xk = np.concatenate([k[rows].float().cpu().numpy(), kn[b:b + 1].float().cpu().numpy()])
        xv = np.concatenate([v[rows].float().cpu().numpy(), vn[b:b + 1].float().cpu().numpy()])
        ck = np.zeros((nblk, H, 16, D), npdt)
        cv = np.zeros((nblk, H, 16, D), npdt)
        sk = np.zeros(nblk, np.float32)
        sv = np.zeros(nblk, np.float32)
        for p in range(T):
            j, t = divmod(p, 16)
            sk[j] = write_token(ck[j], sk[j], t, xk[p])
            sv[j] = write_token(cv[j], sv[j], t, xv[p])
        ids = torch.from_numpy(tables[b][:nblk].astype(np.int64)).to(d)
        np.testing.assert_array_equal(layer.k_pool[ids].cpu().numpy(), ck)
        np.testing.assert_array_equal(layer.v_pool[ids].cpu().numpy(), cv)
        np.testing.assert_array_equal(layer.k_scale[ids].cpu().numpy().view(np.uint32),
                                      sk.view(np.uint32))
        np.testing.assert_array_equal(layer.v_scale[ids].cpu().numpy().view(np.uint32),
                                      sv.view(np.uint32))
        # [nblk, H, 16, D] -> [H, T, D] stored values of the oracle's codes
        Kq = (decode(ck) * sk[:, None, None, None].astype(np.float64)).transpose(1, 0, 2, 3)
        Vq = (decode(cv) * sv[:, None, None, None].astype(np.float64)).transpose(1, 0, 2, 3)
        Kq, Vq = Kq.reshape(H, T, D), Vq.reshape(H, T, D)
        for h in range(H):
            check(got[b, h], decode_row(qh[b, h], Kq[h], Vq[h], w.scale), TOL["f16"],
                  f"codes b={b} h={h}")
            check(got[b, h], decode_row(qh[b, h], xk[:, h], xv[:, h], w.scale), TOL[fmt],
                  f"raw b={b} h={h}")
