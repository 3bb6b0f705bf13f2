"""Benchmark: decode attention over a paged (or contiguous) KV cache on one MI355X.

One step = one decode step of the whole batch through every layer: host slot reservation
(first fit / copy-on-write), block-table and length upload, then per layer the copy-on-write
block copies, the new token's K/V write, decode attention pass 1 (split-context online
softmax) and pass 2 (merge of split sequence-heads). With `--append fused` (the default for
f32/f16 caches) the new token's K/V is stored by pass 1 itself, which takes that row from the
new K/V instead of reading it back; `--append separate` runs the cache writer first (always the
case for 8-bit (e4m3, int8) caches, whose block scale may change, and rolling windows). Inputs are
synthetic and already resident in device memory when timing starts; each step grows every
sequence by one token.

Prints one JSON line. `value` is the HBM throughput of the whole step in GB/s, counting the
algorithmic bytes only (every cached K/V byte read once, block-table entries, q, out, the new
K/V written). `roofline` is for the dominant kernel (attention pass 1), timed with HIP events
recorded on the stream it is launched on. `cpu_baseline` is the CPU oracle timed on one layer.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "paged decode-attention HBM GB/s (% of peak) and decode tokens/s, 1 MI355X"
PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published figure
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 matrix-core peak, AMD's published figure
ELT = {"f32": 4, "f16": 2, "e4m3": 1, "i8": 1}


WORKLOADS = {
    "llama13b-paged": workloads.LLAMA13B_PAGED, "fp8-longctx": workloads.LONGCTX_FP8,
    "llama7b-contig": workloads.LLAMA7B_CONTIG, "tiny-gpt": workloads.TINY_GPT,
    "parallel-sampling": workloads.PARALLEL_SAMPLING,
    "parallel-sampling-cow": workloads.PARALLEL_SAMPLING_COW,
    "gqa8-paged": workloads.GQA8_PAGED, "llama13b-window": workloads.LLAMA13B_WINDOW,
    "llama7b-prefill": workloads.LLAMA7B_PREFILL, "i8-longctx": workloads.LONGCTX_I8,
    "i8-compress": workloads.COMPRESS_I8,
}
SAMPLING = (workloads.PARALLEL_SAMPLING, workloads.PARALLEL_SAMPLING_COW)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama13b-paged",
                    choices=list(WORKLOADS))
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0: model's)")
    ap.add_argument("--append", choices=["auto", "fused", "separate"], default="auto",
                    help="store the new K/V inside attention pass 1 (fused) or with the cache "
                         "writer first (separate); auto = fused unless the cache is 8-bit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU oracle sample: layers of the last step until this many seconds "
                         "(all BLAS threads), then the same layers on one thread")
    ap.add_argument("--time-every", type=int, default=4,
                    help="time attention pass 1 with HIP events on every Nth layer (events "
                         "between launches cost time themselves; 1 times every launch)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the read-ceiling probe of the paged multi-head workloads")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_LOG"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; csv output) "
                         "of this script with --copy-calibration, and print the traffic record")
    ap.add_argument("--graph", action="store_true",
                    help="contiguous workloads (no host work per step): after the eager warm-up, "
                         "capture the timed steps once as a HIP graph (torch.cuda.CUDAGraph) and "
                         "time one replay; the time per launch is then the replay's GPU time over "
                         "its steps x layers, gaps between launches included")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (torch) 3 times; its "
                         "FETCH_SIZE/WRITE_SIZE counters calibrate the HBM traffic figures")
    return ap.parse_args()


class PagedBench:
    """Paged workloads: LLaMA-13B shapes with drawn lengths, or fp8 long context."""

    ORACLE_PER_LAYER = True

    def __init__(self, w: workloads.Workload, steps: int, layers: int, dev, fused: bool):
        import torch

        import kv_cache_attention_kvc_amd as kvc

        self.kvc, self.torch, self.w, self.dev = kvc, torch, w, dev
        self.L = layers
        self.fused = fused
        B, H, D = w.batch, w.heads, w.head_dim
        self.B, self.H, self.D = B, H, D
        self.G = w.extra.get("group", 1)   # query heads per K/V head
        self.W = w.extra.get("window", 0)  # rolling window (0: none)
        if w.ctx:
            lens = np.full(B, w.ctx, dtype=np.int64)
        else:
            lens = workloads.llama13b_lengths(w)
        self.first_lens = lens                        # attended length at the first step
        grow = steps + 1
        nblk = int(sum(workloads.blocks_for(L + grow) for L in lens)) + B
        self.mbps = workloads.blocks_for(int(lens.max()) + grow)
        order = workloads.llama13b_pool_order(nblk, w.seed)
        self.pool = kvc.Pool(nblk, self.mbps, order=order)
        self.seqs = [self.pool.alloc() for _ in range(B)]
        self.layers = [kvc.PagedLayer.empty(nblk, H, D, w.kv_dtype, device=dev, fill=0.0)
                       for _ in range(layers)]
        # prefill: every sequence holds L_b - 1 tokens, written per layer in one call
        slots = np.concatenate([self.pool.append([s], int(L) - 1)[0]
                                for s, L in zip(self.seqs, lens)])
        if self.W:
            self.pool.slide(self.seqs, self.W)
        self._fill(slots)
        self._step_buffers(int(lens.max()) + grow)
        self.lens_now = lens.copy() - 1

    def _fill(self, slots) -> None:
        """Write synthetic K/V rows at `slots` of every layer (one call per layer)."""
        torch, w = self.torch, self.w
        slots_d = torch.from_numpy(slots).to(self.dev)
        for li, layer in enumerate(self.layers):
            k = workloads.torch_normal((len(slots), self.H, self.D), torch.float16, self.dev,
                                       w.seed * 1000 + 2 * li)
            v = workloads.torch_normal((len(slots), self.H, self.D), torch.float16, self.dev,
                                       w.seed * 1000 + 2 * li + 1)
            self.kvc.write_paged(layer, slots_d, k, v)
            del k, v
        torch.cuda.synchronize()

    def _step_buffers(self, max_ctx: int) -> None:
        """Per-step inputs resident in device memory (new K/V and q of every layer), the output,
        the workspace, and a ring of pinned host buffers for the table/length/slot uploads."""
        torch, w, dev, layers = self.torch, self.w, self.dev, self.L
        B, H, D = self.B, self.H, self.D
        Hq = H * self.G
        self.knew = workloads.torch_normal((layers, B, H, D), torch.float16, dev, w.seed * 7 + 1)
        self.vnew = workloads.torch_normal((layers, B, H, D), torch.float16, dev, w.seed * 7 + 2)
        self.q = workloads.torch_normal((layers, B, Hq, D), torch.float16, dev, w.seed * 7 + 3)
        self.out = torch.empty((layers, B, Hq, D), dtype=torch.float16, device=dev)
        self.ws = self.kvc.new_gqa_workspace(B, H, self.G, D, device=dev)
        # a buffer is refilled only after the copy that last read it has executed (the host may
        # run several steps ahead of the GPU)
        self.ring = [(torch.empty((B, self.mbps), dtype=torch.int32, pin_memory=True),
                      torch.empty(B, dtype=torch.int32, pin_memory=True),
                      torch.empty(B, dtype=torch.int64, pin_memory=True),
                      torch.cuda.Event()) for _ in range(4)]
        self.ring_i = 0
        self.tab_d = torch.empty((B, self.mbps), dtype=torch.int32, device=dev)
        self.len_d = torch.empty(B, dtype=torch.int32, device=dev)
        self.slot_d = torch.empty(B, dtype=torch.int64, device=dev)
        self.cow_d = torch.empty((2, B), dtype=torch.int32, device=dev)
        self.max_ctx = max_ctx
        self.scale = float(np.float32(1.0 / math.sqrt(D)))
        self.stream = torch.cuda.current_stream()
        # pass 1 of few, short sequence-heads finishes every row itself: no merge launch then
        self.need_merge = self.kvc.decode_merge_needed(
            True, "f16", w.kv_dtype, B, H, D, self.mbps * 16, max_ctx, G=self.G, window=self.W,
            append=self.fused)

    def step(self, ev=None):
        kvc, torch = self.kvc, self.torch
        slots, src, dst = self.pool.append(self.seqs, 1)
        if self.W:
            self.pool.slide(self.seqs, self.W)
        tab_h, len_h, slot_h, done = self.ring[self.ring_i]
        self.ring_i = (self.ring_i + 1) % len(self.ring)
        done.synchronize()
        self.pool.block_table(self.seqs, out_tables=tab_h.numpy(), out_lens=len_h.numpy())
        slot_h.numpy()[:] = slots
        self.tab_d.copy_(tab_h, non_blocking=True)
        self.len_d.copy_(len_h, non_blocking=True)
        self.slot_d.copy_(slot_h, non_blocking=True)
        done.record(self.stream)
        ncow = len(src)
        if ncow:
            self.cow_d[0, :ncow].copy_(torch.from_numpy(src))
            self.cow_d[1, :ncow].copy_(torch.from_numpy(dst))
        self.lens_now += 1
        for li, layer in enumerate(self.layers):
            if ncow:
                kvc.copy_blocks(layer, self.cow_d[0, :ncow], self.cow_d[1, :ncow])
            if not self.fused:
                kvc.write_paged(layer, self.slot_d, self.knew[li], self.vnew[li])
            if ev is not None:
                ev[0].record(ev[1] + 2 * li, self.stream)
            if self.fused and self.G > 1:
                kvc.append_decode_gqa_partial_paged(self.q[li], layer, self.tab_d, self.len_d,
                                                    self.knew[li], self.vnew[li], self.max_ctx,
                                                    scale=self.scale, out=self.out[li],
                                                    workspace=self.ws)
            elif self.fused:
                kvc.append_decode_partial_paged(self.q[li], layer, self.tab_d, self.len_d,
                                                self.knew[li], self.vnew[li], self.max_ctx,
                                                scale=self.scale, out=self.out[li],
                                                workspace=self.ws)
            elif self.W:
                kvc.decode_window_partial_paged(self.q[li], layer, self.tab_d, self.len_d,
                                                self.max_ctx, self.W, scale=self.scale,
                                                out=self.out[li], workspace=self.ws)
            elif self.G > 1:
                kvc.decode_gqa_partial_paged(self.q[li], layer, self.tab_d, self.len_d,
                                             self.max_ctx, scale=self.scale, out=self.out[li],
                                             workspace=self.ws)
            else:
                kvc.decode_partial_paged(self.q[li], layer, self.tab_d, self.len_d, self.max_ctx,
                                         scale=self.scale, out=self.out[li], workspace=self.ws)
            if ev is not None:
                ev[0].record(ev[1] + 2 * li + 1, self.stream)
            if not self.need_merge:
                continue
            if self.G > 1 or self.W:
                kvc.decode_gqa_merge(self.B, self.H, self.G, self.D, self.out[li], self.ws)
            else:
                kvc.decode_merge(self.B, self.H, self.D, self.out[li], self.ws)

    def bytes_step(self, lens):
        """Algorithmic HBM bytes of one step over all layers, and of one pass-1 launch: every
        attended K/V row read once (the new one from the new-K/V buffer), the new rows written
        once, block tables (and fp8 scales) of the attended blocks, lengths, q and out. The fused
        pass 1 also does the write. With a rolling window only the window's rows and blocks
        count."""
        elt = ELT[self.w.kv_dtype]
        B, H, D = self.B, self.H, self.D
        first = np.maximum(lens - self.W, 0) if self.W else np.zeros_like(lens)
        kv = int((lens - first).sum()) * H * D * 2 * elt
        blocks = int(sum(workloads.blocks_for(L) - int(f) // 16 for L, f in zip(lens, first)))
        q8 = self.w.kv_dtype in ("e4m3", "i8")
        table = blocks * 4 + (blocks * 8 if q8 else 0) + B * 4
        qo = B * H * self.G * D * (2 + 2)
        append = B * H * D * 2 * elt + (B * 8 if q8 else 0)
        pass1 = kv + table + qo + (append if self.fused else 0)
        return (kv + table + qo + append) * self.L, pass1

    def gpu_sample(self):
        return self.out[0]

    def oracle_layer(self, li):
        """The CPU oracle's decode of one layer on the current state (for cpu_baseline and a
        parity spot check): returns (seconds, output [B,H,D], bytes read)."""
        from oracle.caches import PagedCache

        layer = self.layers[li]
        tables, lens = self.pool.block_table(self.seqs)
        first = np.maximum(lens - self.W, 0) if self.W else np.zeros_like(lens)
        ref = PagedCache(layer.num_blocks, self.H, self.D, self.w.kv_dtype)
        ref.K = layer.k_pool.cpu().numpy()
        ref.V = layer.v_pool.cpu().numpy()
        if self.w.kv_dtype in ("e4m3", "i8"):
            ref.k_scale = layer.k_scale.cpu().numpy()
            ref.v_scale = layer.v_scale.cpu().numpy()
        q = self.q[li].float().cpu().numpy()
        t0 = time.perf_counter()
        out = ref.decode(q, tables, lens, self.scale, window=self.W)
        dt = time.perf_counter() - t0
        return dt, out, int((lens - first).sum()) * self.H * self.D * 2 * ELT[self.w.kv_dtype]


    def tile_pieces(self):
        """Pass 1's K/V reads of the current step as (offset, pool pairs): the byte offset of
        every (K/V head, sequence, block) tile in the order of pass 1's work list on a paged
        pool (pair-major: one head of every sequence, then the next head), and each layer's K
        and V pools (None for workloads whose list is not that: rolling windows). The probe's
        wavefronts take consecutive runs of it in launch order; pass 1 also places each XCD's
        runs contiguously, which the probe does not."""
        if self.W:
            return None
        tables, lens = self.pool.block_table(self.seqs)
        tile = 16 * self.D * ELT[self.w.kv_dtype]
        ids = [tables[b][:workloads.blocks_for(int(lens[b]))].astype(np.int64)
               for b in range(len(lens))]
        offs = [(blk * self.H + h) * tile for h in range(self.H) for blk in ids]
        return np.concatenate(offs), tile, [(l.k_pool, l.v_pool) for l in self.layers]


class SamplingBench(PagedBench):
    """Parallel sampling: 8 candidates share one prompt's blocks (the prompt's sequence and 7
    forks, refcount 8), then each step appends one token to every candidate -- copy-on-write of
    the shared partial block at the first step when the prompt ends inside a block -- and attends,
    in every layer. After `generate` steps the candidates are freed and the prompt is taken again
    (first fit in block-id order gives it the same blocks, whose K/V are still in place) and
    forked; that host work is part of the step that follows."""

    def __init__(self, w: workloads.Workload, steps: int, layers: int, dev, fused: bool):
        import torch

        import kv_cache_attention_kvc_amd as kvc

        self.kvc, self.torch, self.w, self.dev = kvc, torch, w, dev
        self.L, self.fused = layers, fused
        self.B, self.H, self.D = w.batch, w.heads, w.head_dim
        self.G, self.W = 1, 0
        self.prompt, self.gen_len = w.extra["prompt"], w.extra["generate"]
        nblk = workloads.blocks_for(self.prompt) + self.B * (workloads.blocks_for(self.gen_len) + 1)
        self.mbps = workloads.blocks_for(self.prompt + self.gen_len)
        self.pool = kvc.Pool(nblk, self.mbps)       # first fit in block-id order
        self.layers = [kvc.PagedLayer.empty(nblk, self.H, self.D, "f16", device=dev, fill=0.0)
                       for _ in range(layers)]
        self.prompt_slots = self._start()
        self._fill(self.prompt_slots)
        self._step_buffers(self.prompt + self.gen_len)
        self.first_lens = np.full(self.B, self.prompt + 1, dtype=np.int64)
        self.lens_now = np.full(self.B, self.prompt, dtype=np.int64)
        self.gen_step = 0
        self.step_ev = None          # (HipEvents, index) per step when timing steps
        self.step_index = []         # generation step of every timed step
        self.cow_per_step = []       # copy-on-write pairs of every timed step
        self.unique_per_step = []    # unique K/V bytes of one layer at every timed step

    def _start(self):
        """The prompt's sequence and its 7 forks; returns the prompt's slots."""
        parent = self.pool.alloc()
        slots = self.pool.append([parent], self.prompt)[0]
        self.seqs = [parent] + [self.pool.fork(parent) for _ in range(self.B - 1)]
        return slots

    def step(self, ev=None):
        if self.gen_step == self.gen_len:
            for s in self.seqs:
                self.pool.free(s)
            slots = self._start()
            if not np.array_equal(slots, self.prompt_slots):
                raise RuntimeError("the prompt did not get its blocks back")
            self.lens_now[:] = self.prompt
            self.gen_step = 0
        before = self.pool.stats()["cow_copies"]
        timed = ev is not None and self.step_ev is not None
        if timed:
            i = ev[1] // (2 * self.L)        # timed step number
            self.step_ev.record(2 * i, self.stream)
        super().step(ev)
        if timed:
            self.step_ev.record(2 * i + 1, self.stream)
            self.cow_per_step.append(self.pool.stats()["cow_copies"] - before)
            self.step_index.append(self.gen_step)
            self.unique_per_step.append(self.unique_bytes())
        self.gen_step += 1

    def unique_bytes(self):
        """Bytes of K/V one layer holds for the current step: every physical block the
        candidates' tables name, once, times its valid slots (shared prompt blocks once)."""
        tables, lens = self.pool.block_table(self.seqs)
        valid = {}
        for b in range(len(lens)):
            L = int(lens[b])
            for j in range(workloads.blocks_for(L)):
                p = int(tables[b][j])
                valid[p] = max(valid.get(p, 0), min(16, L - 16 * j))
        return sum(valid.values()) * self.H * self.D * 2 * ELT["f16"]


class PrefillBench:
    """Prefill: every sequence's whole prompt enters at once. One step = per layer, the prompt's
    K/V written into the paged cache, then causal attention of every prompt row (matrix cores).
    The same slots are rewritten each step."""

    ORACLE_PER_LAYER = False   # the oracle sample is one fixed piece of the last layer

    def tile_pieces(self):
        return None

    def __init__(self, w: workloads.Workload, steps: int, layers: int, dev, fused: bool):
        import torch

        import kv_cache_attention_kvc_amd as kvc

        self.kvc, self.torch, self.w, self.dev, self.L = kvc, torch, w, dev, layers
        B, H, D, T = w.batch, w.heads, w.head_dim, w.extra["prompt"]
        self.B, self.H, self.D, self.T = B, H, D, T
        N = B * workloads.blocks_for(T)
        self.pool = kvc.Pool(N, workloads.blocks_for(T), order=workloads.llama13b_pool_order(N, w.seed))
        self.seqs = [self.pool.alloc() for _ in range(B)]
        slots = np.concatenate([self.pool.append([s], T)[0] for s in self.seqs])
        self.slots = torch.from_numpy(slots).to(dev)
        tables, lens = self.pool.block_table(self.seqs)
        self.tab_d = torch.from_numpy(tables).to(dev)
        self.len_d = torch.from_numpy(lens).to(dev)
        self.qs_d = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * T).to(dev)
        self.layers = [kvc.PagedLayer.empty(N, H, D, w.kv_dtype, device=dev)
                       for _ in range(layers)]
        self.k = [workloads.torch_normal((B * T, H, D), torch.float16, dev, w.seed * 1000 + 3 * li)
                  for li in range(layers)]
        self.v = [workloads.torch_normal((B * T, H, D), torch.float16, dev, w.seed * 1000 + 3 * li + 1)
                  for li in range(layers)]
        self.q = [workloads.torch_normal((B * T, H, D), torch.float16, dev, w.seed * 1000 + 3 * li + 2)
                  for li in range(layers)]
        self.out = torch.empty((B * T, H, D), dtype=torch.float16, device=dev)
        self.scale = w.scale
        self.stream = torch.cuda.current_stream()
        self.first_lens = lens.astype(np.int64)
        self.lens_now = lens.astype(np.int64)

    def step(self, ev=None):
        kvc = self.kvc
        for li, layer in enumerate(self.layers):
            kvc.write_paged(layer, self.slots, self.k[li], self.v[li])
            if ev is not None:
                ev[0].record(ev[1] + 2 * li, self.stream)
            kvc.prefill_paged(self.q[li], layer, self.tab_d, self.qs_d, self.len_d,
                              scale=self.scale, out=self.out)
            if ev is not None:
                ev[0].record(ev[1] + 2 * li + 1, self.stream)

    def flops_launch(self) -> float:
        """Useful flops of one prefill launch: row i of a prompt attends i + 1 positions, with
        2*D flops each for the score and for the weighted value sum."""
        T = self.T
        return self.B * self.H * (T * (T + 1) / 2) * 4 * self.D

    def bytes_step(self, lens):
        """Algorithmic HBM bytes: the K/V written and read once, q read, out written."""
        elt = ELT[self.w.kv_dtype]
        rows = self.B * self.T * self.H * self.D
        kv = rows * 2 * elt
        pass1 = kv + rows * 2 * 2 + self.B * workloads.blocks_for(self.T) * 4
        return (pass1 + kv) * self.L, pass1

    def gpu_sample(self):
        """The GPU rows oracle_layer computes: the first prompt of the last layer."""
        return self.out[:self.T]

    def oracle_layer(self, li):
        """The CPU oracle's prefill of the first prompt of the last layer (a bounded sample; its
        output is still in the output buffer)."""
        from oracle.attention import full_causal

        li = self.L - 1
        k = self.k[li][:self.T].float().cpu().numpy()
        v = self.v[li][:self.T].float().cpu().numpy()
        q = self.q[li][:self.T].float().cpu().numpy()
        t0 = time.perf_counter()
        ref = np.stack([full_causal(q[:, h], k[:, h], v[:, h], self.scale) for h in range(self.H)],
                       axis=1)
        dt = time.perf_counter() - t0
        return dt, ref, self.T * self.H * self.D * 2 * ELT[self.w.kv_dtype]


class CompressBench:
    """Whole-cache 8-bit compression: every sequence's fp16 blocks re-encoded into an int8 pool
    with fresh per-block scales, one kvc_compress_blocks launch per layer (the same blocks each
    step; the destination is overwritten)."""

    ORACLE_PER_LAYER = False   # the oracle sample is one fixed piece of the last layer

    def tile_pieces(self):
        return None

    def __init__(self, w: workloads.Workload, steps: int, layers: int, dev, fused: bool):
        import torch

        import kv_cache_attention_kvc_amd as kvc

        self.kvc, self.torch, self.w, self.dev, self.L = kvc, torch, w, dev, layers
        B, H, D, T = w.batch, w.heads, w.head_dim, w.ctx
        self.B, self.H, self.D, self.T = B, H, D, T
        N = B * workloads.blocks_for(T)
        self.pool = kvc.Pool(N, workloads.blocks_for(T), order=workloads.llama13b_pool_order(N, w.seed))
        self.seqs = [self.pool.alloc() for _ in range(B)]
        slots = np.concatenate([self.pool.append([s], T)[0] for s in self.seqs])
        slots_d = torch.from_numpy(slots).to(dev)
        src_dt = w.extra["compress_from"]
        self.src = [kvc.PagedLayer.empty(N, H, D, src_dt, device=dev) for _ in range(layers)]
        self.dst = [kvc.PagedLayer.empty(N, H, D, w.kv_dtype, device=dev) for _ in range(layers)]
        for li, layer in enumerate(self.src):
            k = workloads.torch_normal((len(slots), H, D), torch.float16, dev, w.seed * 1000 + 2 * li)
            v = workloads.torch_normal((len(slots), H, D), torch.float16, dev, w.seed * 1000 + 2 * li + 1)
            kvc.write_paged(layer, slots_d, k, v)
            del k, v
        # every block of every sequence, in table order; a block holds min(16, T - 16j) slots
        tables, lens = self.pool.block_table(self.seqs)
        ids, nval = [], []
        for b in range(B):
            for j in range(workloads.blocks_for(int(lens[b]))):
                ids.append(int(tables[b][j]))
                nval.append(min(16, int(lens[b]) - 16 * j))
        self.ids = np.array(ids, dtype=np.int32)
        self.nval = np.array(nval, dtype=np.int32)
        self.ids_d = torch.from_numpy(self.ids).to(dev)
        self.nval_d = torch.from_numpy(self.nval).to(dev)
        self.stream = torch.cuda.current_stream()
        self.first_lens = lens.astype(np.int64)
        self.lens_now = lens.astype(np.int64)
        torch.cuda.synchronize()

    def step(self, ev=None):
        for li in range(self.L):
            if ev is not None:
                ev[0].record(ev[1] + 2 * li, self.stream)
            self.kvc.compress_blocks(self.src[li], self.dst[li], self.ids_d, self.ids_d,
                                     self.nval_d)
            if ev is not None:
                ev[0].record(ev[1] + 2 * li + 1, self.stream)

    def bytes_step(self, lens):
        """Algorithmic HBM bytes of one launch: the valid source rows of K and V read (fp16),
        every destination slot of K and V written (one byte each), the two scales per block
        written, and the block ids and counts read."""
        src_elt = ELT[self.w.extra["compress_from"]]
        rows = int(self.nval.sum()) * self.H * self.D
        nblk = len(self.ids)
        per = rows * 2 * src_elt + nblk * 16 * self.H * self.D * 2 * ELT[self.w.kv_dtype] \
            + nblk * (2 * 4 + 2 * 4)
        return per * self.L, per

    SAMPLE = 2048  # blocks of the last layer the CPU oracle compresses (about 15 s)

    def gpu_sample(self):
        """Stored values (codes x block scale) of the first SAMPLE blocks of the last layer."""
        dst = self.dst[-1]
        idx = self.ids_d[:self.SAMPLE].long()
        k = dst.k_pool[idx].float() * dst.k_scale[idx].view(-1, 1, 1, 1)
        v = dst.v_pool[idx].float() * dst.v_scale[idx].view(-1, 1, 1, 1)
        return self.torch.stack([k, v])

    def oracle_layer(self, li):
        """The CPU oracle's compression of the first SAMPLE blocks of the last layer."""
        from oracle.codecs import compress_block, e4m3_decode, i8_decode

        src = self.src[-1]
        idx = self.ids_d[:self.SAMPLE].long()
        ks = src.k_pool[idx].float().cpu().numpy()
        vs = src.v_pool[idx].float().cpu().numpy()
        n = self.nval[:self.SAMPLE]
        t0 = time.perf_counter()
        out = np.zeros((2,) + ks.shape)
        for i in range(len(n)):
            for j, x in enumerate((ks[i], vs[i])):
                c, s = compress_block(x, int(n[i]), self.w.kv_dtype)
                dec = e4m3_decode(c) if self.w.kv_dtype == "e4m3" else i8_decode(c)
                out[j, i] = dec * np.float64(s)
        dt = time.perf_counter() - t0
        nbytes = int(n.sum()) * self.H * self.D * 2 * ELT[self.w.extra["compress_from"]]
        return dt, out, nbytes


class HipEvents:
    """HIP timing events recorded on a stream, created with hipEventDisableSystemFence: a timing
    event then skips the system-scope cache write-back and invalidate that default events do,
    which would otherwise be timed too and would slow the kernels that follow."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes

        self.n = n
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            self.ev.append(e)

    def record(self, i: int, stream) -> None:
        rc = self.hip.hipEventRecord(self.ev[i], self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


class SampledEvents:
    """HipEvents recorded only around the launches of every `every`-th layer: event index i
    belongs to layer (i // 2) % layers; the others' records are skipped."""

    def __init__(self, layers: int, steps: int, every: int):
        self.layers, self.steps, self.every = layers, steps, max(1, every)
        self.ev = HipEvents(2 * layers * steps)

    def sampled(self, li: int) -> bool:
        return li % self.every == 0

    def record(self, i: int, stream) -> None:
        if self.sampled((i // 2) % self.layers):
            self.ev.record(i, stream)

    def launch_ms(self):
        """Pass-1 launch times of the sampled layers, [steps, sampled layers]."""
        return np.array([[self.ev.elapsed_ms(2 * (self.layers * s + li),
                                             2 * (self.layers * s + li) + 1)
                          for li in range(self.layers) if self.sampled(li)]
                         for s in range(self.steps)])

    def close(self) -> None:
        self.ev.close()


class ContigBench:
    """Contiguous [B, H, S_max, D] caches. LLaMA-7B shapes: every step appends one token per
    sequence at position ctx-1 (overwriting, so each step attends exactly ctx positions) and
    attends. Tiny char-GPT: a 16-token prefill, then each step appends at the next position and
    attends (context 17 .. 256)."""

    ORACLE_PER_LAYER = True

    def __init__(self, w: workloads.Workload, steps: int, layers: int, dev, fused: bool):
        import torch

        import kv_cache_attention_kvc_amd as kvc

        self.kvc, self.torch, self.w, self.dev, self.L = kvc, torch, w, dev, layers
        self.fused = fused
        B, H, D, S = w.batch, w.heads, w.head_dim, w.s_max
        self.B, self.H, self.D, self.S = B, H, D, S
        self.growing = "prefill" in w.extra
        pre = w.extra["prefill"] if self.growing else w.ctx - 1
        if self.growing and pre + steps > S:
            raise SystemExit(f"at most {S - pre} steps for {w.name}")
        td = torch.float32 if w.kv_dtype == "f32" else torch.float16
        self.kc, self.vc = [], []
        zeros = torch.zeros(B, dtype=torch.int32, device=dev)
        for li in range(layers):
            k = torch.empty((B, H, S, D), dtype=td, device=dev)
            v = torch.empty_like(k)
            kn = workloads.torch_normal((B, pre, H, D), td, dev, w.seed * 1000 + 2 * li)
            vn = workloads.torch_normal((B, pre, H, D), td, dev, w.seed * 1000 + 2 * li + 1)
            kvc.append_contig(k, v, zeros, kn, vn)
            del kn, vn
            self.kc.append(k)
            self.vc.append(v)
        torch.cuda.synchronize()
        self.knew = workloads.torch_normal((layers, B, 1, H, D), td, dev, w.seed * 7 + 1)
        self.vnew = workloads.torch_normal((layers, B, 1, H, D), td, dev, w.seed * 7 + 2)
        self.knew3 = self.knew.view(layers, B, H, D)      # the same rows, [B, H, D] per layer
        self.vnew3 = self.vnew.view(layers, B, H, D)
        self.q = workloads.torch_normal((layers, B, H, D), td, dev, w.seed * 7 + 3)
        self.out = torch.empty((layers, B, H, D), dtype=td, device=dev)
        self.ws = kvc.new_workspace(B, H, D, device=dev)
        self.pos = pre                      # next position written
        self.pos_d = torch.full((B,), pre, dtype=torch.int32, device=dev)
        self.len_d = torch.full((B,), pre + 1, dtype=torch.int32, device=dev)
        if self.growing:
            # every step's write positions and attended lengths, resident before timing
            p = torch.arange(pre, pre + steps, dtype=torch.int32, device=dev)
            self.pos_all = p[:, None].expand(steps, B).contiguous()
            self.len_all = (self.pos_all + 1).contiguous()
            self.step_i = 0
        self.scale = w.scale
        self.stream = torch.cuda.current_stream()
        self.lens_now = np.full(B, pre, dtype=np.int64)

    def step(self, ev=None):
        kvc = self.kvc
        pos_d, len_d = self.pos_d, self.len_d
        if self.growing:
            pos_d, len_d = self.pos_all[self.step_i], self.len_all[self.step_i]
            self.step_i += 1
        self.lens_now[:] = self.pos + 1
        for li in range(self.L):
            if not self.fused:
                kvc.append_contig(self.kc[li], self.vc[li], pos_d, self.knew[li], self.vnew[li])
            if ev is not None:
                ev[0].record(ev[1] + 2 * li, self.stream)
            if self.fused and self.growing:
                # short contexts: one launch (pass 1 combines each sequence-head itself and
                # the merge launch is skipped when nothing is left for it)
                kvc.append_decode_contig(self.q[li], self.kc[li], self.vc[li], len_d,
                                         self.knew3[li], self.vnew3[li], self.pos + 1,
                                         scale=self.scale, out=self.out[li], workspace=self.ws)
                if ev is not None:
                    ev[0].record(ev[1] + 2 * li + 1, self.stream)
                continue
            if self.fused:
                kvc.append_decode_partial_contig(self.q[li], self.kc[li], self.vc[li],
                                                 len_d, self.knew3[li], self.vnew3[li],
                                                 self.pos + 1, scale=self.scale,
                                                 out=self.out[li], workspace=self.ws)
            else:
                kvc.decode_partial_contig(self.q[li], self.kc[li], self.vc[li], len_d,
                                          self.pos + 1, scale=self.scale, out=self.out[li],
                                          workspace=self.ws)
            if ev is not None:
                ev[0].record(ev[1] + 2 * li + 1, self.stream)
            kvc.decode_merge(self.B, self.H, self.D, self.out[li], self.ws)
        if self.growing:
            self.pos += 1

    def bytes_step(self, lens):
        elt = ELT[self.w.kv_dtype]
        B, H, D = self.B, self.H, self.D
        kv = int(lens.sum()) * H * D * 2 * elt
        qo = B * H * D * 2 * elt
        append = B * H * D * 2 * elt
        pass1 = kv + qo + B * 4 + (append if self.fused else 0)
        return (kv + qo + B * 4 + append) * self.L, pass1

    def gpu_sample(self):
        return self.out[0]

    def tile_pieces(self):
        """Pass 1's K/V reads of the current step: the byte offset of every (sequence, head,
        16-position tile) in work-list order, and each layer's K and V caches."""
        row = self.D * ELT[self.w.kv_dtype]
        offs = [((b * self.H + h) * self.S + 16 * j) * row
                for b in range(self.B) for h in range(self.H)
                for j in range(workloads.blocks_for(int(self.lens_now[b])))]
        return (np.array(offs, dtype=np.int64), 16 * row,
                [(self.kc[li], self.vc[li]) for li in range(self.L)])

    def oracle_layer(self, li):
        from oracle.caches import ContigCache

        ref = ContigCache(self.B, self.H, self.S, self.D, self.w.kv_dtype)
        ref.K = self.kc[li].cpu().numpy()
        ref.V = self.vc[li].cpu().numpy()
        q = self.q[li].float().cpu().numpy()
        lens = self.lens_now.copy()
        t0 = time.perf_counter()
        out = ref.decode(q, lens, self.scale)
        dt = time.perf_counter() - t0
        return dt, out, int(lens.sum()) * self.H * self.D * 2 * ELT[self.w.kv_dtype]


KV_CODE = {"f32": 0, "f16": 1, "e4m3": 2, "i8": 3}


def _b(x: bool) -> str:
    return "true" if x else "false"


def kernel_match(w: workloads.Workload, fused: bool) -> str:
    """The dominant kernel's instance as rocprofv3 names it (template arguments as printed)."""
    if w is workloads.LLAMA7B_PREFILL:
        return "prefill_kernel<true, 128>"
    if w is workloads.COMPRESS_I8:
        return "compress_f16_stream_kernel<3"
    G = w.extra.get("group", 1)
    paged = w.kind == "paged"
    win = "window" in w.extra
    if G == 1:
        return (f"decode_partial_kernel<{_b(paged)}, {KV_CODE[w.kv_dtype]}, {w.head_dim}, "
                f"{_b(w.q_dtype == 'f16')}, 1, {_b(win)}>")
    return (f"decode_partial_mfma_kernel<{_b(paged)}, {KV_CODE[w.kv_dtype]}, {w.head_dim}, "
            f"{_b(win)}, {_b(fused)}>")


def kernel_name(w: workloads.Workload) -> str:
    """The pass-1 kernel the workload runs: the vector kernel for multi-head attention, the
    matrix-core kernel (up to 16 query heads per wavefront, a divisor of the group) for shared
    K/V heads with fp16 queries."""
    G = w.extra.get("group", 1)
    win = ", rolling window" if "window" in w.extra else ""
    if w is workloads.LLAMA7B_PREFILL:
        return f"kvc::prefill_kernel<{w.kind}, {w.head_dim}> (causal prefill on the matrix cores)"
    if w is workloads.COMPRESS_I8:
        return (f"kvc::compress_blocks_kernel<{w.extra['compress_from']} source, {w.kv_dtype}> "
                "(one-shot 8-bit block compression)")
    if G == 1:
        return (f"kvc::decode_partial_kernel<{w.kind}, {w.kv_dtype}, {w.head_dim}{win}> "
                "(attention pass 1)")
    gq = max(d for d in range(1, 17) if G % d == 0)
    return (f"kvc::decode_partial_mfma_kernel<{w.kind}, {w.kv_dtype}, {w.head_dim}{win}> (attention "
            f"pass 1 on the matrix cores, {gq} query heads per wavefront)")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


# committed HBM traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE), one per workload
PROFILE_TAG = {
    workloads.LLAMA13B_PAGED.name: "decode_partial_paged_f16_llama13b",
    workloads.LLAMA7B_CONTIG.name: "decode_partial_contig_f16_llama7b",
    workloads.LONGCTX_FP8.name: "decode_partial_paged_e4m3_longctx",
    workloads.GQA8_PAGED.name: "decode_partial_mfma_paged_f16_gqa8",
    workloads.PARALLEL_SAMPLING.name: "decode_partial_paged_f16_parallel_sampling",
    workloads.PARALLEL_SAMPLING_COW.name: "decode_partial_paged_f16_parallel_sampling_cow",
    workloads.COMPRESS_I8.name: "compress_f16_to_i8_longctx",
    workloads.LLAMA13B_WINDOW.name: "decode_partial_paged_f16_llama13b_window1024",
    workloads.LONGCTX_I8.name: "decode_partial_paged_i8_longctx",
    workloads.LLAMA7B_PREFILL.name: "prefill_paged_f16_llama7b_b4x2048",
}


def traffic_file(w: workloads.Workload):
    tag = PROFILE_TAG.get(w.name)
    return os.path.join(ROOT, "profiles", f"{tag}_traffic.txt") if tag else None


def source_hash(path: str) -> str:
    """First 16 hex digits of the sha256 of a kernel source."""
    import hashlib

    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def workload_source(w: workloads.Workload) -> str:
    """The HIP source of the workload's dominant kernel."""
    name = ("kvc_prefill.hip" if w is workloads.LLAMA7B_PREFILL else
            "kvc_write.hip" if w is workloads.COMPRESS_I8 else "kvc_decode.hip")
    return os.path.join(ROOT, "kv_cache_attention_kvc_amd", "csrc", name)


def pmc_summary(fetch_dir: str, write_dir: str, bench_log: str) -> dict:
    """HBM bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), each scaled by what the same counter reads for a plain 1 GiB device copy.
    Only the timed launches count (the last steps x layers dispatches of the kernel), so the
    figure describes the same launches as the bench line's `achieved`."""
    import csv
    import glob

    rec = None
    for ln in open(bench_log):
        if ln.startswith("{"):
            rec = json.loads(ln)
    roof, cfg = rec["roofline"], rec["config"]
    match = roof["kernel_match"]
    n_timed = rec["steps"] * cfg["layers"]

    def rows(d):
        (f,) = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        return list(csv.DictReader(open(f)))

    def dispatch_key(r):
        for k in ("Dispatch_Id", "Correlation_Id"):
            if k in r and r[k] != "":
                return int(r[k])
        return 0

    def per_kernel(rs):
        v = sorted(((dispatch_key(r), float(r["Counter_Value"])) for r in rs
                    if match in r["Kernel_Name"]))
        v = [x for _, x in v][-n_timed:]
        return sum(v) / len(v), len(v)

    def copy_kib(rs):
        v = sorted(float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"]
                   and int(r["Grid_Size"]) >= 65536)
        return v[-1]

    fr, wr = rows(fetch_dir), rows(write_dir)
    cal = float(1 << 30)
    f_fac = cal / (copy_kib(fr) * 1024)
    w_fac = cal / (copy_kib(wr) * 1024)
    fk, nf = per_kernel(fr)
    wk, nw = per_kernel(wr)
    alg = roof["algorithmic_bytes_per_launch"]
    fetch_b = fk * 1024 * f_fac
    write_b = wk * 1024 * w_fac
    out = {"kernel": match, "workload": cfg["workload"], "steps": rec["steps"],
           "warmup": rec["warmup"], "layers": cfg["layers"],
           "source_sha256_16": roof["kernel_source_sha256_16"], "append": cfg["append"],
           "dispatches_averaged": [nf, nw],
           "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
           "fetch_scale": round(f_fac, 5), "write_scale": round(w_fac, 5),
           "fetch_bytes": int(fetch_b), "write_bytes": int(write_b),
           "traffic_bytes": int(fetch_b + write_b),
           "algorithmic_bytes_per_launch_same_run": alg,
           "traffic_over_algorithmic": round((fetch_b + write_b) / alg, 4)}
    if "sampling" in rec:
        u = rec["sampling"]["unique_bytes_per_launch"]
        out["unique_bytes_per_launch_same_run"] = u
        out["fetch_over_unique"] = round(fetch_b / u, 4)
    return out


def measured_traffic(w: workloads.Workload, path: str, steps: int, warmup: int, layers: int):
    """Traffic per launch of the dominant kernel from the committed counter record, if that
    record was taken over the same launches as this run (workload, steps, warm-up, layers, append
    path) on the current kernel source; else None."""
    f = traffic_file(w)
    if not f:
        return None
    try:
        for ln in open(f):
            if ln.startswith("{"):
                rec = json.loads(ln)
                same = (rec.get("workload") == w.name and rec.get("steps") == steps
                        and rec.get("warmup") == warmup and rec.get("layers") == layers
                        and rec.get("append") == path
                        and rec.get("source_sha256_16") == source_hash(workload_source(w)))
                return rec["traffic_bytes"] if same else None
    except OSError:
        pass
    return None


def cpu_baseline(bench, layers: int, budget_s: float):
    """The CPU oracle timed on the last step: layer after layer until budget_s seconds have
    passed (all BLAS threads), then the same layers on one thread. Returns (record fields,
    total seconds, layer count, the oracle's output of layer 0)."""
    from threadpoolctl import threadpool_limits

    t_all, nbytes, calls, ref0 = 0.0, 0, [], None
    n = layers if bench.ORACLE_PER_LAYER else 1
    # layer after layer (round again over the layers when a pass takes less than the budget)
    while t_all < budget_s and len(calls) < 100000:
        li = len(calls) % n
        dt, ref, nb = bench.oracle_layer(li)
        if ref0 is None:
            ref0 = ref
        t_all += dt
        nbytes += nb
        calls.append(li)
        if not bench.ORACLE_PER_LAYER and len(calls) >= 1 and t_all >= budget_s / 4:
            break
    with threadpool_limits(limits=1):
        t_one = sum(bench.oracle_layer(li)[0] for li in calls)
    threads = blas_threads()
    rec = {"value": round(nbytes / t_all / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "value_1thread": round(nbytes / t_one / 1e9, 4),
           "cpu_count": os.cpu_count(), "blas_threads": threads,
           "seconds": round(t_all, 3), "seconds_1thread": round(t_one, 3),
           "oracle_calls": len(calls)}
    return rec, (t_all, len(calls), len(set(calls))), ref0


def read_ceiling(bench, p1_achieved: float):
    """The read ceiling of pass 1's access pattern: kvc_read_pieces over exactly the K/V tiles
    of the last step in work-list order, each layer's pools in turn (as the timed run reads
    them), at 8, 12 and 16 wavefronts per CU; and a sequential read of the same bytes from the
    start of each layer's pools. HIP events on the launch stream, three passes over the layers,
    median launch time."""
    import torch

    import kv_cache_attention_kvc_amd as kvc

    pieces = bench.tile_pieces()
    if pieces is None:
        return None
    offs, tile, pools = pieces
    n = len(offs)
    nbytes = n * 2 * tile
    dev = bench.dev
    patterns = {"pass1_tiles": torch.from_numpy(offs).to(dev),
                "sequential": torch.arange(n, dtype=torch.int64, device=dev) * tile}
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    res, by_wpc = {}, {}
    reps = 3
    for name, off_d in patterns.items():
        best = None
        for wpc in (8, 12, 16):
            ev = HipEvents(2 * reps * len(pools))
            k = 0
            for _ in range(reps):
                for kp, vp in pools:
                    ev.record(2 * k, bench.stream)
                    kvc.read_pieces(kp, off_d, tile, wpc, sink, b=vp)
                    ev.record(2 * k + 1, bench.stream)
                    k += 1
            torch.cuda.synchronize()
            t = float(np.median([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(k)])) / 1e3
            ev.close()
            gbs = nbytes / t / 1e9
            if name == "pass1_tiles":
                by_wpc[str(wpc)] = round(gbs, 1)
            if best is None or gbs > best[0]:
                best = (gbs, wpc, t)
        res[name] = best
    return {"gbs": round(res["pass1_tiles"][0], 1),
            "pattern": "pass 1's K/V tiles of the last step, work-list order, one layer per launch",
            "waves_per_cu": res["pass1_tiles"][1],
            "gbs_by_waves_per_cu": by_wpc,
            "sequential_gbs": round(res["sequential"][0], 1),
            "bytes_per_launch": nbytes,
            "pass1_over_ceiling": round(p1_achieved / res["pass1_tiles"][0], 4)}


def main():
    args = parse()
    if args.pmc_summary:
        print(json.dumps(pmc_summary(*args.pmc_summary)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: decode attention "
              "here runs on a single MI355X, and sharding across GPUs is not implemented",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    layers = args.layers or w.layers
    K, W = args.steps, args.warmup
    if w is workloads.TINY_GPT and K + W > w.extra["decode_steps"]:
        K, W = w.extra["decode_steps"], 0
    print(f"[bench] setting up {w.name}: {layers} layers, {K} timed + {W} warm-up steps",
          file=sys.stderr, flush=True)
    separate = (w.kv_dtype in ("e4m3", "i8") or "window" in w.extra
                or w is workloads.LLAMA7B_PREFILL)
    fused = args.append == "fused" or (args.append == "auto" and not separate)
    if fused and separate:
        print("--append fused: 8-bit caches and rolling windows take the separate writer",
              file=sys.stderr)
        sys.exit(2)
    path = "fused" if fused else "separate"
    prefill = w is workloads.LLAMA7B_PREFILL
    compress = w is workloads.COMPRESS_I8
    sampling = w in SAMPLING
    cls = (PrefillBench if prefill else CompressBench if compress else
           SamplingBench if sampling else PagedBench if w.kind == "paged" else ContigBench)
    bench = cls(w, K + W, layers, dev, fused)
    for _ in range(W):
        bench.step()
    torch.cuda.synchronize()
    print("[bench] warm-up done", file=sys.stderr, flush=True)

    if sampling:
        bench.step_ev = HipEvents(2 * K)
        bench.gen_step = bench.gen_len     # the timed steps start a fresh generation
    total_bytes = 0
    pass1_bytes, unique = [], []
    if args.graph:
        if cls is not ContigBench:
            print("--graph: only contiguous workloads, which do no host work per step, are "
                  "captured", file=sys.stderr)
            sys.exit(2)
        # the K timed steps captured once (nothing runs during capture), then one replay timed
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for s in range(K):
                bench.step(None)
                b_all, b_p1 = bench.bytes_step(bench.lens_now)
                total_bytes += b_all
                pass1_bytes.append(b_p1)
        rep = HipEvents(2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rep.record(0, torch.cuda.current_stream())
        graph.replay()
        rep.record(1, torch.cuda.current_stream())
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        elapsed = t1 - t0
        p1_ms = np.full((K, layers), rep.elapsed_ms(0, 1) / (K * layers))
        rep.close()
        del graph
    else:
        evs = SampledEvents(layers, K, args.time_every)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            bench.step((evs, 2 * layers * s))
            b_all, b_p1 = bench.bytes_step(bench.lens_now)
            total_bytes += b_all
            pass1_bytes.append(b_p1)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        elapsed = t1 - t0
        p1_ms = evs.launch_ms()   # [K, sampled layers]
        evs.close()
    p1_avg_s = float(p1_ms.mean()) / 1e3
    p1_bytes_avg = float(np.mean(pass1_bytes))
    achieved = p1_bytes_avg / p1_avg_s / 1e9
    value = total_bytes / elapsed / 1e9
    traffic = measured_traffic(w, path, K, W, layers)
    if prefill:
        # compute-bound: the roofline is the matrix cores' fp16 peak over the useful flops
        roof = {"bound": "mfma", "achieved": round(bench.flops_launch() / p1_avg_s / 1e12, 1),
                "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(bench.flops_launch() / p1_avg_s / 1e12 / PEAK_F16_TFLOPS, 4),
                "traffic": None, "flops_per_launch": bench.flops_launch()}
        tokens = w.batch * bench.T * K
    elif compress:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic}
        tokens = w.batch * bench.T * K  # cached tokens compressed (in every layer) per step
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic}
        tokens = w.batch * K
    print(f"[bench] timed: {elapsed * 1e3 / K:.3f} ms/step, pass 1 {p1_avg_s * 1e6:.1f} us/launch",
          file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic: N(0,1) K/V/q, seeded; lengths and pool order seeded",
        "config": {
            "workload": w.name, "batch": w.batch, "heads": w.heads * w.extra.get("group", 1),
            "kv_heads": w.heads, "head_dim": w.head_dim,
            "layers": layers, "block_size": 16, "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype,
            "ctx_first_step": ("U[%d,%d] mean %.1f" % (w.ctx_lo, w.ctx_hi, bench.first_lens.mean()))
            if w.ctx_hi else (w.extra["prefill"] + 1 if "prefill" in w.extra else
                              w.extra["prompt"] + 1 if sampling else w.ctx),
            "ctx_growth_per_step": 0 if w in (workloads.LLAMA7B_CONTIG, workloads.LLAMA7B_PREFILL,
                                              workloads.COMPRESS_I8) else 1,
            "window": w.extra.get("window", 0),
            "append": path,
            **({"launch": "hip graph of the timed steps, one replay"} if args.graph else {}),
            **({"merge_launch": bool(bench.need_merge)} if hasattr(bench, "need_merge") else {}),
        },
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "tokens_per_s": round(tokens / elapsed, 1),
        "roofline": {
            "kernel": kernel_name(w),
            "kernel_match": kernel_match(w, fused),
            **roof,
            "avg_launch_us": round(p1_avg_s * 1e6, 2),
            "timed_launches": int(p1_ms.size),
            **({"launch_timing": "one graph replay's GPU time over steps x layers (pass 1, the "
                                 "merge where it runs, and the gaps between launches)"}
               if args.graph else {}),
            "algorithmic_bytes_per_launch": int(p1_bytes_avg),
            "kernel_source": os.path.basename(workload_source(w)),
            "kernel_source_sha256_16": source_hash(workload_source(w)),
        },
    }
    if traffic is not None:
        line["roofline"]["traffic_over_algorithmic"] = round(traffic / p1_bytes_avg, 4)
    if sampling:
        step_us = np.array([bench.step_ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)]) * 1e3
        bench.step_ev.close()
        idx = np.array(bench.step_index)
        line["sampling"] = {
            "candidates": w.batch, "prompt": bench.prompt, "generate": bench.gen_len,
            "cow_copies_per_generation": int(sum(c for c, i in zip(bench.cow_per_step, idx)
                                                 if i == 0) / max(1, int((idx == 0).sum()))),
            "blocks_used_last_step": bench.pool.stats()["used"],
            "first_step_us": round(float(step_us[idx == 0].mean()), 1) if (idx == 0).any() else None,
            "other_steps_median_us": round(float(np.median(step_us[idx != 0])), 1),
            "first_step_extra_us": (round(float(step_us[idx == 0].mean() - np.median(step_us[idx != 0])),
                                          1) if (idx == 0).any() else None),
            "logical_gbs": round(value, 1),
            "unique_bytes_per_launch": int(np.mean(bench.unique_per_step)),
            "logical_bytes_per_launch_last_step": int(pass1_bytes[-1]),
        }
    if not args.no_ceiling and not prefill and not compress and not sampling:
        print("[bench] read ceiling", file=sys.stderr, flush=True)
        ceil = read_ceiling(bench, achieved)
        if ceil is not None:
            line["roofline"]["ceiling"] = ceil
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle", file=sys.stderr, flush=True)
        rec, (t_all, ncalls, used), ref = cpu_baseline(bench, layers, args.cpu_seconds)
        got = bench.gpu_sample().float().cpu().numpy()
        per_layer = t_all / ncalls
        rec["sample"] = (
            (f"the first prompt of the last layer: {bench.T} rows x {w.heads} heads, causal; "
             f"{bench.T / (per_layer * layers):.3f} prefill tokens/s over {layers} layers")
            if prefill else
            (f"the first {bench.SAMPLE} blocks of the last layer (K and V)") if compress else
            (f"{ncalls} oracle decodes of layers 0..{used - 1} of the last step: all "
             f"{w.batch} sequences x {w.heads * w.extra.get('group', 1)} query heads, "
             f"{int(bench.lens_now.sum())} positions per layer; "
             f"{w.batch / (per_layer * layers):.3f} tokens/s over {layers} layers (all threads)"))
        line["cpu_baseline"] = rec
        # a sanity check of the timed run, not a parity claim: the oracle reads the cache as the
        # library stored it (the parity tests build every oracle input from the generated data)
        line["spot_check"] = {"max_abs_err": float(np.abs(got - ref).max()),
                              "oracle_input": "the cache as stored on the device"}
    if args.copy_calibration:
        a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = 1 << 30
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
