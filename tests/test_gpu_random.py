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
    if window:
        got = kvc.decode_window_paged(qd, layer, td, tld, max(lens), window, scale=scale_of(D))
    elif G > 1:
        got = kvc.decode_gqa_paged(qd, layer, td, tld, max(lens), scale=scale_of(D))
    else:
        got = kvc.decode_attn_paged(qd, layer, td, tld, max(lens), scale=scale_of(D))
    torch.cuda.synchronize()
    want = ref.decode(q, tables, tl, scale_of(D), window=window)
    check(got.float().cpu().numpy(), want, TOL["f32"] if dtype == "f32" else TOL["f16"],
          f"seed={seed}")
    # empty sequences give zero rows
    for b, L in enumerate(lens):
        if L == 0:
            assert got[b].float().abs().sum().item() == 0.0
