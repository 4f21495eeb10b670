#!/usr/bin/env python3
"""Benchmark of decode-phase paged attention on one MI355X.

A step is one pass of the whole hot path over one batch: for every layer,
the cache write of the batch's new tokens followed by paged decode attention
(plus, for the shared-prompt workload, the copy-on-write block copies).
Inputs are synthetic, seeded and already resident in HBM when timing starts.

Prints ONE JSON line: achieved HBM GB/s over the step (algorithmic bytes /
time) as ``value``, decode tokens/s (sequences x layers per second), the
dominant kernel's roofline fraction against MI355X's 8 TB/s, and the CPU
oracle's throughput on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "paged decode attention: achieved HBM GB/s (% of peak) + decode tokens/s, 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- byte accounting
def attention_bytes(ctx, num_seqs, num_heads, num_kv_heads, head_dim, kv_bytes, q_bytes,
                    block_size, unique_tokens=None):
    """Algorithmic bytes of one decode launch: every live K/V token once (shared
    prompt blocks once), q and out once, the used table entries and lengths."""
    tokens = int(np.sum(ctx)) if unique_tokens is None else int(unique_tokens)
    kv = tokens * 2 * num_kv_heads * head_dim * kv_bytes
    qo = 2 * num_seqs * num_heads * head_dim * q_bytes
    tables = int(np.sum((np.asarray(ctx, np.int64) + block_size - 1) // block_size)) * 4
    return kv + qo + tables + 4 * num_seqs


def write_bytes(num_tokens, num_kv_heads, head_dim, src_bytes, kv_bytes):
    return num_tokens * (2 * num_kv_heads * head_dim * (src_bytes + kv_bytes) + 8)


# ---------------------------------------------------------------- workloads
class Workload:
    """A decode step over ``L`` layers, each with its own pools in HBM.

    Subclasses fill: S, H, Hkv, D, bs, L, ctx, kv_dtype, q_dtype, layers (list of
    dicts of device tensors: k_pool, v_pool, k_new, v_new, q, out), tables,
    ctx_t, slots, scale, k_scale, v_scale, attn_bytes, write_bytes.
    """
    pairs = None            # copy-on-write pairs applied each step (shared-prompt batch)
    k_scale = v_scale = 1.0

    def finish(self, pa, torch, partition_size, max_ctx):
        self.pa, self.torch = pa, torch
        self.partition_size = partition_size
        self.max_ctx = int(max_ctx)
        ws = pa.paged_attention_workspace_size(self.S, self.H, self.Hkv, self.D, self.max_ctx,
                                               partition_size)
        self.ws = pa.new_workspace(ws, "cuda")
        for d in self.layers:
            d.setdefault("out", torch.empty_like(d["q"]))
        self.step_bytes = self.L * (self.attn_bytes + self.write_bytes) + \
            (0 if self.pairs is None else self.L * len(self.pairs) * 2 * 2 * self.block_bytes)
        self.seq_layers_per_step = self.S * self.L

    def decode(self, l):
        d = self.layers[l]
        self.pa.paged_attention_decode(d["out"], d["q"], d["k_pool"], d["v_pool"], self.tables,
                                       self.ctx_t, max_context_len=self.max_ctx, scale=self.scale,
                                       k_scale=self.k_scale, v_scale=self.v_scale,
                                       partition_size=self.partition_size, workspace=self.ws)

    def step(self):
        if self.pairs is not None and len(self.pairs):
            self.pa.copy_blocks([d["k_pool"] for d in self.layers],
                                [d["v_pool"] for d in self.layers], self.pairs_d)
        for l in range(self.L):
            d = self.layers[l]
            self.pa.kv_cache_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], self.slots,
                                   k_scale=self.k_scale, v_scale=self.v_scale)
            self.decode(l)

    def config(self):
        return {"workload": self.name, "num_seqs": self.S, "num_layers": self.L,
                "num_heads": self.H, "num_kv_heads": self.Hkv, "head_dim": self.D,
                "block_size": self.bs, "kv_dtype": self.kv_dtype, "q_dtype": self.q_dtype,
                "context_lens": self.ctx_desc, "partition_size": self.partition_size}

    def roofline(self, call_ms):
        """Decode is bound by HBM: algorithmic bytes per call over the call time."""
        achieved = self.attn_bytes / (call_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "algorithmic_bytes_per_launch": self.attn_bytes}

    def cpu_inputs(self, l, s):
        """Host copies of what the oracle needs for sequence s of layer l: the
        sequence's blocks (a local table 0..n-1), its new K/V and its query."""
        torch = self.torch
        d = self.layers[l]
        n = int(self.ctx[s])
        nblk = (n + self.bs - 1) // self.bs
        if not hasattr(self, "_tables_np"):
            self._tables_np = self.tables.cpu().numpy()
        idx = torch.from_numpy(self._tables_np[s, :nblk].astype(np.int64)).cuda()
        kp, vp = raw_np(d["k_pool"][idx]), raw_np(d["v_pool"][idx])
        pos = n - 1
        slot = np.array([(pos // self.bs) * self.bs + pos % self.bs])
        return dict(kp=kp, vp=vp, kn=raw_np(d["k_new"][s:s + 1]), vn=raw_np(d["v_new"][s:s + 1]),
                    q=raw_np(d["q"][s:s + 1]), slot=slot, n=n,
                    local=np.arange(nblk, dtype=np.int32)[None, :])

    def cpu_run(self, oracle, x):
        """The oracle as it stands: cache write, then attention, for one sequence-layer."""
        oracle.kv_write(x["kp"], x["vp"], self.kv_dtype, x["kn"], x["vn"], self.q_dtype, x["slot"],
                        self.bs, self.k_scale, self.v_scale)
        oracle.paged_attention(x["q"], self.q_dtype, x["kp"], x["vp"], self.kv_dtype, x["local"],
                               [x["n"]], self.bs, self.scale, self.k_scale, self.v_scale)

    def cpu_sample(self, oracle, budget_s, cores):
        """Oracle throughput on a bounded sample: sequence-layers, longest contexts
        first, layer after layer, run `cores` at a time on a thread pool (NumPy
        releases the interpreter lock in its array loops).  Only the oracle calls
        are timed; copying each batch's inputs to the host is not."""
        import concurrent.futures as cf
        order = np.argsort(-self.ctx, kind="stable")
        work = [(l, int(s)) for l in range(self.L) for s in order]
        done, secs, kv_bytes, i = 0, 0.0, 0, 0
        with cf.ThreadPoolExecutor(cores) as ex:
            while i < len(work) and secs < budget_s:
                batch = work[i:i + cores]
                i += len(batch)
                xs = [self.cpu_inputs(l, s) for l, s in batch]
                t0 = time.perf_counter()
                list(ex.map(lambda x: self.cpu_run(oracle, x), xs))
                secs += time.perf_counter() - t0
                done += len(batch)
                kv_bytes += sum(x["n"] for x in xs) * 2 * self.Hkv * self.D * ELEM[self.kv_dtype]
        layers = len({l for l, _ in work[:i]})
        sample = (f"{done} sequence-layers (all {self.H} heads each) from {layers} layer(s), longest "
                  f"contexts first, {kv_bytes / 1e6:.1f} MB of K/V, {cores} at a time")
        return {"value": round(done / secs, 3), "unit": "seq-layers/s", "cores": cores,
                "kind": "oracle", "sample": sample, "cpu_model": cpu_model(),
                "host_cpus": os.cpu_count(), "seconds": round(secs, 2),
                "kv_gbs_equivalent": round(kv_bytes / secs / 1e9, 3)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_cores():
    """Threads for the oracle baseline: every core this process may run on, at
    most 16 (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1, "int8": 1}


def raw_np(t):
    """Device tensor -> numpy storage array (bf16 as raw uint16)."""
    t = t.detach().cpu()
    if t.dtype.__str__() == "torch.bfloat16":
        import torch
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload_case(case, torch):
    import workloads as W
    def dev(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dt == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.cuda()
    return {"k_pool": dev(case.k_pool, case.kv_dtype), "v_pool": dev(case.v_pool, case.kv_dtype),
            "k_new": dev(case.k_new, case.q_dtype), "v_new": dev(case.v_new, case.q_dtype),
            "q": dev(case.q, case.q_dtype)}


class Llama7B(Workload):
    """Llama-2-7B-shaped decode step over all 32 layers: 64 sequences at context
    4096, 32 heads x 128, block size 16, fp16 cache, 17,408-block pool per layer
    (4.25 GiB of K+V per layer, 136 GiB in all), one block table for all layers."""
    name = "llama2-7b decode step, 32 layers, fp16 KV"

    def __init__(self, pa, W, torch, partition_size, args):
        self.S, self.H, self.Hkv, self.D, self.bs, self.NB, self.L = 64, 32, 32, 128, 16, 17408, 32
        self.kv_dtype = self.q_dtype = "f16"
        self.ctx = np.full(self.S, 4096, dtype=np.int32)
        self.ctx_desc = "all 4096"
        self.layers = []
        t0 = time.time()
        for l in range(self.L):
            d = W.device_pool_case(f"llama7b_l{l}", "llama7b", num_seqs=self.S, num_heads=self.H,
                                   num_kv_heads=self.Hkv, head_dim=self.D, block_size=self.bs,
                                   context_lens=self.ctx, kv_dtype="f16", num_blocks=self.NB,
                                   layer=l, place_layer=0)
            self.layers.append(d)
        torch.cuda.synchronize()
        log(f"generated {self.L} layers of pools in {time.time() - t0:.1f}s")
        d0 = self.layers[0]
        self.tables = torch.from_numpy(d0["tables"]).cuda()
        self.ctx_t = torch.from_numpy(self.ctx).cuda()
        self.slots = torch.from_numpy(d0["slots"]).cuda()
        self.scale = d0["scale"]
        self.attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 2, 2, self.bs)
        self.write_bytes = write_bytes(self.S, self.Hkv, self.D, 2, 2)
        self.finish(pa, torch, partition_size, 4096)

    def config(self):
        c = super().config()
        c["num_blocks_per_layer"] = self.NB
        return c


class HostLayers(Workload):
    """Workloads small enough to generate on the host: layer 0 comes from the
    seeded generator, the other layers are copies of it in their own memory
    (distinct addresses, so no layer's K/V can be served from another's cache
    lines; the 256 MB last-level cache cannot hold the step's working set)."""

    def place(self, torch, case, L):
        self.case = case
        self.S, self.H, self.Hkv, self.D = case.num_seqs, case.num_heads, case.num_kv_heads, case.head_dim
        self.bs, self.NB, self.L = case.block_size, case.num_blocks, L
        self.kv_dtype, self.q_dtype = case.kv_dtype, case.q_dtype
        self.ctx = case.context_lens.astype(np.int32)
        self.scale, self.k_scale, self.v_scale = case.scale, case.k_scale, case.v_scale
        base = upload_case(case, torch)
        self.layers = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(L - 1)]
        self.tables = torch.from_numpy(case.block_tables.astype(np.int32)).cuda()
        self.ctx_t = torch.from_numpy(self.ctx).cuda()
        self.slots = torch.from_numpy(case.slot_mapping.astype(np.int64)).cuda()
        self.block_bytes = self.Hkv * self.bs * self.D * ELEM[self.kv_dtype]
        self.write_bytes = write_bytes(self.S, self.Hkv, self.D, ELEM[self.q_dtype], ELEM[self.kv_dtype])
        torch.cuda.synchronize()


class Opt13B(HostLayers):
    """OPT-13B-shaped layer (40 heads x 128, fp16, block 16, 30 sequences with
    log-normal contexts, 1,000-block pool), stepped over OPT-13B's 40 layers."""
    name = "opt-13b decode step, 40 layers, fp16 KV"

    def __init__(self, pa, W, torch, partition_size, args):
        case = W.opt13b_case()
        self.place(torch, case, 40)
        self.ctx_desc = f"log-normal median 300, sum {int(self.ctx.sum())}, max {int(self.ctx.max())}"
        self.attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 2, 2, self.bs)
        self.finish(pa, torch, partition_size, self.ctx.max())


class Falcon7B(HostLayers):
    """Falcon-7B-shaped MQA layer: 71 query heads share 1 KV head of 64, fp8 e4m3
    cache with per-tensor scales, fp16 q/out, 256 sequences with contexts uniform
    in 1..2048, stepped over Falcon-7B's 32 layers."""
    name = "falcon-7b decode step, 32 layers, fp8 KV (MQA)"

    def __init__(self, pa, W, torch, partition_size, args):
        bs = args.block_size or 16
        ctx = W.falcon7b_lengths(256)
        case = W.make_decode_case(f"falcon7b_bs{bs}", "falcon7b", num_seqs=256, num_heads=71,
                                  num_kv_heads=1, head_dim=64, block_size=bs, context_lens=ctx,
                                  kv_dtype="fp8_e4m3", q_dtype="f16",
                                  num_blocks=W.falcon7b_num_blocks(ctx, bs))
        self.place(torch, case, 32)
        self.ctx_desc = f"uniform 1..2048, sum {int(self.ctx.sum())}"
        self.attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 1, 2, self.bs)
        self.finish(pa, torch, partition_size, self.ctx.max())


class Llama70B(HostLayers):
    """Llama-2-70B-shaped GQA layer (64 query heads over 8 KV heads of 128, bf16,
    block 16): 96 independent sequences with log-normal contexts plus 8 groups of
    4 parallel samples that share a 520-token prompt; every step applies the
    copy-on-write block copies, the cache write and attention, over L layers."""
    name = "llama2-70b GQA decode step, bf16 KV, shared-prompt samples"

    def __init__(self, pa, W, torch, partition_size, args):
        NB = 12288
        spec = W.llama70b_spec()
        alloc = pa.BlockAllocator(NB, 16, W.free_order("llama70b", NB))
        case, pairs = W.shared_prompt_case(alloc, spec, num_blocks=NB)
        self.place(torch, case, args.layers or 8)
        self.pairs = pairs
        self.pairs_d = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).cuda()
        P, n_ind = spec.prompt_len, len(spec.independent_ctx)
        # shared full prompt blocks are read once; every sample owns its copied last block
        full = (P // 16) * 16
        shared_extra = (spec.samples - 1) * full * spec.groups
        self.unique_tokens = int(self.ctx.sum()) - shared_extra
        self.ctx_desc = (f"96 log-normal median 1024 (128..8192) + 8x4 samples at {P + 1}; "
                         f"sum {int(self.ctx.sum())}, unique {self.unique_tokens}")
        self.attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 2, 2, self.bs,
                                          unique_tokens=self.unique_tokens)
        self.logical_attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 2, 2,
                                                  self.bs)
        self.finish(pa, torch, partition_size, self.ctx.max())


class Llama7BInt8(HostLayers):
    """Llama-2-7B-shaped layer with a group-wise int8 cache (32 heads x 128, block
    16, one float32 scale per token and KV head for K and for V), fp16 q/out:
    16 sequences at context 2048, 8 layers in their own memory."""
    name = "llama2-7b-shaped decode step, int8 KV (group-wise scales)"

    def __init__(self, pa, W, torch, partition_size, args):
        case = W.make_int8_case("llama7b_int8", "llama7b", num_seqs=16, num_heads=32,
                                num_kv_heads=32, head_dim=128, block_size=16,
                                context_lens=[2048] * 16, q_dtype="f16", spare_blocks=16)
        self.place(torch, case, args.layers or 8)
        ks = torch.from_numpy(case.k_scales).cuda()
        vs = torch.from_numpy(case.v_scales).cuda()
        for i, d in enumerate(self.layers):
            d["k_scales"] = ks if i == 0 else ks.clone()
            d["v_scales"] = vs if i == 0 else vs.clone()
        torch.cuda.synchronize()
        self.ctx_desc = "all 2048"
        tokens = int(self.ctx.sum())
        # codes once, plus each token's K and V scale per KV head
        self.attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 1, 2, self.bs) + \
            tokens * 2 * self.Hkv * 4
        self.write_bytes = write_bytes(self.S, self.Hkv, self.D, 2, 1) + self.S * 2 * self.Hkv * 4
        self.finish(pa, torch, partition_size, self.ctx.max())

    def decode(self, l):
        d = self.layers[l]
        self.pa.paged_attention_decode_int8(d["out"], d["q"], d["k_pool"], d["v_pool"],
                                            d["k_scales"], d["v_scales"], self.tables, self.ctx_t,
                                            max_context_len=self.max_ctx, scale=self.scale,
                                            partition_size=self.partition_size, workspace=self.ws)

    def step(self):
        for l in range(self.L):
            d = self.layers[l]
            self.pa.kv_cache_write_int8(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"],
                                        d["k_scales"], d["v_scales"], self.slots)
            self.decode(l)

    def cpu_inputs(self, l, s):
        x = super().cpu_inputs(l, s)
        d = self.layers[l]
        nblk = x["local"].shape[1]
        idx = self.torch.from_numpy(self._tables_np[s, :nblk].astype(np.int64)).cuda()
        x["ks"], x["vs"] = d["k_scales"][idx].cpu().numpy(), d["v_scales"][idx].cpu().numpy()
        return x

    def cpu_run(self, oracle, x):
        oracle.kv_write_int8(x["kp"], x["vp"], x["ks"], x["vs"], x["kn"], x["vn"], self.q_dtype,
                             x["slot"], self.bs)
        oracle.paged_attention(x["q"], self.q_dtype, x["kp"], x["vp"], "int8", x["local"],
                               [x["n"]], self.bs, self.scale, x["ks"], x["vs"])


class Tiny(HostLayers):
    """The tiny fp32 case: 4 sequences, contexts {5,10,3,16}, 2 heads of 64, block 4."""
    name = "tiny fp32 decode step, 1 layer"

    def __init__(self, pa, W, torch, partition_size, args):
        self.place(torch, W.tiny_case(), 1)
        self.ctx_desc = "5, 10, 3, 16"
        self.attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 4, 4, self.bs)
        self.finish(pa, torch, partition_size, self.ctx.max())


PEAK_MFMA_F16_TFLOPS = 2500.0     # MI355X dense fp16/bf16 matrix-core peak


class Llama7BPrefill(Workload):
    """Llama-2-7B-shaped chunked prefill over 32 layers: 8 sequences with 0, 512, ...,
    3,584 tokens cached and a 512-token chunk each (contexts 512..4096), 32 heads x
    128, fp16, block 16.  A step writes the chunk's K/V and runs causal multi-token
    attention in every layer (layers are copies of layer 0 in their own memory).
    Bound by the matrix cores: flops = 4 x (visible query-key pairs) x heads x head_dim."""
    name = "llama2-7b chunked prefill step, 32 layers, fp16 KV, 512-token chunks"
    bound = "mfma"

    def __init__(self, pa, W, torch, partition_size, args):
        case = W.llama7b_prefill_case()
        self.case = case
        self.pa, self.torch = pa, torch
        self.S, self.H, self.Hkv, self.D = case.num_seqs, case.num_heads, case.num_kv_heads, case.head_dim
        self.bs, self.NB, self.L = case.block_size, case.num_blocks, args.layers or 32
        self.kv_dtype, self.q_dtype = case.kv_dtype, case.q_dtype
        self.scale = case.scale
        self.ctx = case.context_lens.astype(np.int32)
        self.partition_size = 0
        base = upload_case(case, torch)
        self.layers = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(self.L - 1)]
        for d in self.layers:
            d["out"] = torch.empty_like(d["q"])
        self.tables = torch.from_numpy(case.block_tables.astype(np.int32)).cuda()
        self.ctx_t = torch.from_numpy(self.ctx).cuda()
        self.qs = torch.from_numpy(case.query_start.astype(np.int32)).cuda()
        self.slots = torch.from_numpy(case.slot_mapping.astype(np.int64)).cuda()
        T = case.num_tokens
        pairs = 0
        for s in range(self.S):
            n, ql = int(self.ctx[s]), int(case.query_start[s + 1] - case.query_start[s])
            pairs += ql * (n - ql) + ql * (ql + 1) // 2
        self.pairs = None
        self.visible_pairs = pairs
        self.flops = 4 * pairs * self.H * self.D
        self.attn_bytes = int(self.ctx.sum()) * 2 * self.Hkv * self.D * 2 + 2 * T * self.H * self.D * 2
        self.write_bytes = write_bytes(T, self.Hkv, self.D, 2, 2)
        self.step_bytes = self.L * (self.attn_bytes + self.write_bytes)
        self.seq_layers_per_step = T * self.L          # query tokens x layers
        torch.cuda.synchronize()

    def decode(self, l):
        d = self.layers[l]
        self.pa.paged_attention_prefill(d["out"], d["q"], d["k_pool"], d["v_pool"], self.tables,
                                        self.ctx_t, self.qs, max_query_len=self.case.max_query_len,
                                        scale=self.scale)

    def step(self):
        for l in range(self.L):
            d = self.layers[l]
            self.pa.kv_cache_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], self.slots)
            self.decode(l)

    def roofline(self, call_ms):
        achieved = self.flops / (call_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_MFMA_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4),
                "flops_per_launch": self.flops}

    def config(self):
        return {"workload": self.name, "num_seqs": self.S, "num_layers": self.L,
                "num_heads": self.H, "num_kv_heads": self.Hkv, "head_dim": self.D,
                "block_size": self.bs, "kv_dtype": self.kv_dtype, "q_dtype": self.q_dtype,
                "cached_tokens": [int(x) for x in self.ctx - 512], "chunk_tokens": 512,
                "visible_query_key_pairs": self.visible_pairs}

    def cpu_inputs(self, l, s):
        """Host copies for 8 query rows of sequence s of layer l spread over its chunk
        (the oracle computes only those rows)."""
        torch = self.torch
        d = self.layers[l]
        case = self.case
        n = int(self.ctx[s])
        nblk = (n + self.bs - 1) // self.bs
        idx = torch.from_numpy(case.block_tables[s, :nblk].astype(np.int64)).cuda()
        r0, r1 = int(case.query_start[s]), int(case.query_start[s + 1])
        rows = np.linspace(0, r1 - r0 - 1, 8).astype(int)
        return dict(kp=raw_np(d["k_pool"][idx]), vp=raw_np(d["v_pool"][idx]),
                    kn=raw_np(d["k_new"][r0:r1]), vn=raw_np(d["v_new"][r0:r1]),
                    q=raw_np(d["q"][r0:r1]), n=n, ql=r1 - r0, rows=rows,
                    slot=self._local_slots(s, nblk),
                    local=np.arange(nblk, dtype=np.int32)[None, :])

    def _local_slots(self, s, nblk):
        """The chunk's slots renumbered for the copied blocks (local table 0..nblk-1)."""
        case = self.case
        r0, r1 = int(case.query_start[s]), int(case.query_start[s + 1])
        phys = case.block_tables[s, :nblk]
        where = {int(b): i for i, b in enumerate(phys)}
        sl = case.slot_mapping[r0:r1]
        return np.array([where[int(x) // self.bs] * self.bs + int(x) % self.bs for x in sl], np.int64)

    def cpu_run(self, oracle, x):
        oracle.kv_write(x["kp"], x["vp"], self.kv_dtype, x["kn"], x["vn"], self.q_dtype, x["slot"],
                        self.bs)
        oracle.paged_prefill(x["q"], self.q_dtype, x["kp"], x["vp"], self.kv_dtype, x["local"],
                             [x["n"]], [0, x["ql"]], self.bs, self.scale, rows=x["rows"])

    def cpu_sample(self, oracle, budget_s, cores):
        """Oracle throughput in query rows per second: 8 rows of each sequence-layer
        (spread over its chunk, so over the whole range of visible lengths), longest
        contexts first, `cores` sequence-layers at a time on a thread pool."""
        import concurrent.futures as cf
        order = np.argsort(-self.ctx, kind="stable")
        work = [(l, int(s)) for l in range(self.L) for s in order]
        rows, secs, i = 0, 0.0, 0
        with cf.ThreadPoolExecutor(cores) as ex:
            while i < len(work) and secs < budget_s:
                batch = work[i:i + cores]
                i += len(batch)
                xs = [self.cpu_inputs(l, s) for l, s in batch]
                t0 = time.perf_counter()
                list(ex.map(lambda x: self.cpu_run(oracle, x), xs))
                secs += time.perf_counter() - t0
                rows += 8 * len(batch)
        return {"value": round(rows / secs, 3), "unit": "query-token-layers/s", "cores": cores,
                "kind": "oracle", "sample": f"{rows} query rows (8 per sequence-layer, spread over "
                f"each chunk), longest contexts first, {cores} sequence-layers at a time",
                "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "seconds": round(secs, 2)}


# launch configuration per workload: the fastest measured on MI355X (uniform
# long contexts: one pass per (sequence, head); ragged batches: balanced split)
DEFAULT_PARTITION = {"llama7b": 0, "opt13b": -1, "falcon7b": -1, "llama70b": -1, "tiny": 0,
                     "llama7b_prefill": 0, "llama7b_int8": 512}

WORKLOADS = {"llama7b": Llama7B, "opt13b": Opt13B, "falcon7b": Falcon7B, "llama70b": Llama70B,
             "tiny": Tiny, "llama7b_prefill": Llama7BPrefill, "llama7b_int8": Llama7BInt8}


def read_traffic(workload, partition_size, block_size):
    """HBM traffic per launch of the dominant kernel from the committed counter
    summary of the same workload, launch mode and block size, if the kernel
    sources are unchanged since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.traffic.txt"))):
        kv = {}
        for line in open(path):
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if kv.get("workload") != workload or "partition_size" not in kv or \
                int(kv["partition_size"]) != partition_size or \
                int(kv.get("block_size", "0")) != block_size:
            continue
        h = hashlib.sha256()
        try:
            for src in kv["sources"].split():
                with open(os.path.join(ROOT, src), "rb") as f:
                    h.update(f.read())
        except OSError:                 # a source of the profiled build is gone
            continue
        if h.hexdigest() == kv["source_sha256"]:
            return int(float(kv["traffic_bytes"])), os.path.basename(path)
    return None, None


def calibrate_copy(pa, torch, mib):
    """One copy_blocks launch moving exactly `mib` MiB (read) + `mib` MiB (write):
    64 pairs of blocks of mib/64 MiB each (f16 pool of 2*64+ blocks)."""
    heads = max(1, mib * 1024 * 1024 // 64 // (256 * 128 * 2))       # 64 KiB per (head) row
    shape = (130, heads, 256, 128)                                     # block = heads x 64 KiB
    kpool = torch.zeros(shape, dtype=torch.float16, device="cuda")
    vpool = torch.zeros(shape, dtype=torch.float16, device="cuda")
    pairs = np.stack([np.arange(64), np.arange(64, 128)], axis=1).astype(np.int32)
    pa.copy_blocks([kpool], [vpool], pairs)
    torch.cuda.synchronize()
    log(f"calibration copy: {mib} MiB read + {mib} MiB written per pool, K and V pools")


# ---------------------------------------------------------------- allocator study (host only)
class ReserveAhead:
    """A contiguous-reservation policy of the kind paging replaces (KV 缓存与分页注意力
    §04-§05): every admitted request reserves one contiguous run of token slots up
    front, placed first-fit in a linear slot space (so gaps between runs are the
    external fragments); `reserve(final_len)` gives the run length."""

    def __init__(self, capacity, reserve):
        self.capacity, self.reserve = capacity, reserve
        self.runs = {}                     # request -> (start, length)

    def admit(self, rid, first_len, final_len):
        size = self.reserve(final_len)
        pos = 0
        for start, length in sorted(self.runs.values()):
            if start - pos >= size:
                break
            pos = max(pos, start + length)
        if pos + size > self.capacity:
            return False
        self.runs[rid] = (pos, size)
        return True

    def grow_all(self, rids):              # each run already holds its whole request
        return True

    def free(self, rid):
        del self.runs[rid]

    def reserved(self):
        return sum(length for _, length in self.runs.values())


class Paged:
    """The library's block allocator: blocks taken as tokens arrive (§06-§07)."""

    def __init__(self, pa, capacity, block_size):
        self.a = pa.BlockAllocator(capacity // block_size, block_size)
        self.bs, self.pa = block_size, pa

    def admit(self, rid, first_len, final_len):
        try:
            self.a.add_seq(rid, first_len)
            return True
        except self.pa.PagedAttnError:
            return False

    def grow_all(self, rids):              # one slot for each, all or none
        if not rids:
            return True
        try:
            self.a.append_slots(rids)
            return True
        except self.pa.PagedAttnError:
            return False

    def free(self, rid):
        self.a.free_seq(rid)

    def reserved(self):
        return self.a.stats()["used_blocks"] * self.bs


def serve_trace(policy, prompts, finals, max_rounds=200000):
    """Requests queued first come first served; each round admits from the head of
    the queue while the policy finds room (a request's prompt lands at once; no
    admission in a round that followed a preemption), then every running request
    writes one token; when that needs room the policy cannot find, the latest
    admitted request gives way (all of its memory: §09) and goes back to the head
    of the queue to start again, until the rest fit.  Readouts: memory holding
    tokens over memory reserved (mean over rounds), concurrent requests (max and
    mean), rounds to finish."""
    queue = list(range(len(prompts)))
    running, written = [], {}
    util, conc, rounds = [], [], 0
    preempted = False
    while (queue or running) and rounds < max_rounds:
        rounds += 1
        while queue and not preempted and policy.admit(queue[0], prompts[queue[0]], finals[queue[0]]):
            rid = queue.pop(0)
            running.append(rid)
            written[rid] = prompts[rid]
        preempted = False
        while True:
            growing = [r for r in running if written[r] < finals[r]]
            if policy.grow_all(growing):
                break
            late = running.pop()                       # latest admitted gives way
            policy.free(late)
            queue.insert(0, late)
            preempted = True
        for r in running:
            written[r] = min(finals[r], written[r] + 1)
        conc.append(len(running))
        res = policy.reserved()
        util.append(sum(written[r] for r in running) / res if res else 1.0)
        done = [r for r in running if written[r] >= finals[r]]
        for rid in done:
            policy.free(rid)
        running = [r for r in running if written[r] < finals[r]]
    return {"utilisation": round(float(np.mean(util)), 4), "max_concurrent": int(max(conc)),
            "mean_concurrent": round(float(np.mean(conc)), 2), "rounds": rounds}


def allocator_study(pa):
    """Utilisation of KV memory by block size and by reservation policy, on seeded
    synthetic traces (host only, the library's allocator for the paged policies).

    * The pages' toy machine (KV 缓存与分页注意力 §14): 176 token slots, 40
      requests of 1..20 tokens (uniform), one token per round; blocks of 1, 2, 4,
      8 or 16 tokens against reserving 20 slots per request.
    * An OPT-13B-sized cache (§03: 12 GB, about 15,700 tokens) serving 400
      requests of log-normal prompt (median 160) and output (median 240) lengths,
      at most 2,048 tokens: blocks of 16 against reserving the maximum, the next
      power of two of the final length, or exactly the final length (the three
      reservation policies of §05)."""
    rng = np.random.default_rng(20230914)
    toy_final = rng.integers(1, 21, size=40)
    toy = {f"block_{bs}": serve_trace(Paged(pa, 176, bs), [1] * 40, toy_final.tolist())
           for bs in (1, 2, 4, 8, 16)}
    toy["reserve_20"] = serve_trace(ReserveAhead(176, lambda f: 20), [1] * 40, toy_final.tolist())
    cap, max_len = 15700, 2048
    prompt = np.clip(np.rint(rng.lognormal(np.log(160), 0.9, 400)), 1, 1024).astype(int)
    out = np.clip(np.rint(rng.lognormal(np.log(240), 0.9, 400)), 1, max_len).astype(int)
    final = np.minimum(prompt + out, max_len)
    pow2 = lambda f: min(max_len, 1 << int(np.ceil(np.log2(max(f, 1)))))
    big = {"paged_block_16": serve_trace(Paged(pa, cap - cap % 16, 16), prompt.tolist(), final.tolist()),
           "reserve_max": serve_trace(ReserveAhead(cap, lambda f: max_len), prompt.tolist(), final.tolist()),
           "reserve_pow2": serve_trace(ReserveAhead(cap, pow2), prompt.tolist(), final.tolist()),
           "reserve_exact": serve_trace(ReserveAhead(cap, lambda f: f), prompt.tolist(), final.tolist())}
    return {"toy_176_slots": toy, "opt13b_15700_tokens": big}


# ---------------------------------------------------------------- main
def reference_read_gbs(torch, pa, mib=2048, reps=10):
    """The library's streaming-read probe over `mib` MiB (the decode kernels' 16-byte
    non-temporal loads, nothing else): the read rate this device reaches, beside the
    8 TB/s denominator.  Measured before the workload's pools are allocated."""
    n = mib << 20
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(pa.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    pa.stream_read(buf, sink)
    torch.cuda.synchronize()
    gbs = 0.0
    for _ in range(3):          # the best of three timings: a ceiling, not an average
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            pa.stream_read(buf, sink)
        b.record()
        torch.cuda.synchronize()
        gbs = max(gbs, float(n) * reps / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf, sink
    torch.cuda.empty_cache()
    return gbs


def reference_copy_gbs(torch, mib=512, reps=10):
    """Device-to-device copy of `mib` MiB with the runtime's copy (read + write bytes
    per second): the bandwidth a plain streaming kernel reaches on this device,
    shown beside the 8 TB/s denominator.  Measured before the workload's pools
    are allocated, and freed again."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2.0 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def measure(wl, torch, steps, warmup, decode_iters, graph=True, singles=True):
    """Time `steps` whole steps (after `warmup`), then the decode call alone back
    to back over the layers, then (optionally) single calls between their own
    events.  Graphs are replayed unless `graph` is false."""
    step_fn = wl.step
    decode_fn = lambda: [wl.decode(l) for l in range(wl.L)]
    for _ in range(max(1, warmup)):
        step_fn()
    torch.cuda.synchronize()
    graphs = []
    if graph:
        g_step, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            wl.step()
        with torch.cuda.graph(g_dec):
            decode_fn()
        graphs = [g_step, g_dec]
        step_fn, decode_fn = g_step.replay, g_dec.replay
        for _ in range(max(1, warmup)):
            step_fn()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step_fn()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps
    rounds = max(1, decode_iters // wl.L)
    start.record()
    for _ in range(rounds):
        decode_fn()
    end.record()
    torch.cuda.synchronize()
    decode_ms = start.elapsed_time(end) / (rounds * wl.L)
    spread = None
    if singles:
        times = []
        for i in range(max(10, min(60, decode_iters))):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            wl.decode(i % wl.L)
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        spread = [round(float(np.percentile(times, q)), 2) for q in (10, 50, 90)]
    del graphs
    return ms_per_step, decode_ms, spread


def config_entry(key, wl, torch, oracle, args, cpu_seconds, cores):
    """Measurements of one workload for the per-config list of the bench line."""
    ms, dec_ms, spread = measure(wl, torch, args.steps, args.warmup, args.decode_iters,
                                 graph=not args.no_graph)
    roof = wl.roofline(dec_ms)
    traffic, src = read_traffic(key, wl.partition_size, wl.bs)
    att = {"avg_launch_us": round(dec_ms * 1e3, 2), **roof,
           "single_call_us_p10_p50_p90": spread, "traffic": traffic,
           "traffic_ratio": None if traffic is None else round(traffic / wl.attn_bytes, 4),
           "traffic_source": src}
    if hasattr(wl, "logical_attn_bytes"):
        att["logical_bytes_per_launch"] = wl.logical_attn_bytes
    e = {"workload": key, "config": wl.config(), "ms_per_step": round(ms, 4),
         "step_gbs": round(wl.step_bytes / (ms * 1e-3) / 1e9, 1),
         "tokens_per_s": round(wl.seq_layers_per_step / (ms * 1e-3), 1),
         "tokens": "query tokens x layers" if roof["bound"] == "mfma" else "sequences x layers",
         "attention": att}
    log(f"[{key} bs{wl.bs}] {ms:.3f} ms/step, attention {dec_ms * 1e3:.1f} us "
        f"({roof['achieved']} {roof['unit']}, {roof['frac']:.3f} of peak)")
    if cpu_seconds > 0:
        e["cpu_baseline"] = wl.cpu_sample(oracle, cpu_seconds, cores)
        log(f"[{key}] cpu oracle: {e['cpu_baseline']['value']} {e['cpu_baseline']['unit']} on {cores} threads")
    return e


# every configuration of the workload set, measured after the headline one
CONFIG_SET = [("tiny", {}), ("opt13b", {}), ("llama70b", {}), ("falcon7b", {"block_size": 8}),
              ("falcon7b", {"block_size": 16}), ("falcon7b", {"block_size": 32}),
              ("falcon7b", {"block_size": 64}), ("llama7b_prefill", {}), ("llama7b_int8", {})]


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b", choices=sorted(WORKLOADS))
    ap.add_argument("--partition-size", type=int, default=None,
                    help="0 single pass, > 0 split-context partitions, -1 balanced split "
                         "(default: the fastest measured for the workload)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU-oracle baseline sample (0 = skip)")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="CPU-oracle budget for each entry of the per-config list")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure the chosen workload only (no per-config list)")
    ap.add_argument("--decode-iters", type=int, default=64)
    ap.add_argument("--block-size", type=int, default=0, help="falcon7b: block size (default 16)")
    ap.add_argument("--layers", type=int, default=0, help="llama70b: layers per step (default 8)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch eagerly instead of replaying a captured HIP graph")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain copy of this many MiB (copy_blocks kernel) so that "
                         "HBM counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_129_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        calibrate_copy(pa, torch, args.calibrate_copy_mib)
    copy_gbs = reference_copy_gbs(torch)
    read_gbs = reference_read_gbs(torch, pa)
    log(f"reference device-to-device copy: {copy_gbs:.0f} GB/s (read + write); "
        f"streaming read: {read_gbs:.0f} GB/s")
    if args.partition_size is None:
        args.partition_size = DEFAULT_PARTITION[args.workload]
    wl = WORKLOADS[args.workload](pa, W, torch, args.partition_size, args)
    ms_per_step, decode_ms, spread = measure(wl, torch, args.steps, args.warmup,
                                             args.decode_iters, graph=not args.no_graph)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    roof = wl.roofline(decode_ms)
    log(f"attention: {decode_ms * 1e3:.1f} us per launch, {roof['achieved']} {roof['unit']}")
    log(f"single calls: p10 {spread[0]} p50 {spread[1]} p90 {spread[2]} us")

    value = wl.step_bytes / (ms_per_step * 1e-3) / 1e9
    traffic, traffic_src = read_traffic(args.workload, args.partition_size, wl.bs)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": wl.config(),
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "decode_tokens_per_s": round(wl.seq_layers_per_step / (ms_per_step * 1e-3), 1),
        "roofline": {**roof, "traffic": traffic,
                     "kernel": "paged_attention_prefill" if roof["bound"] == "mfma"
                     else "paged_attention_decode",
                     "avg_launch_us": round(decode_ms * 1e3, 2),
                     "single_call_us_p10_p50_p90": spread,
                     "traffic_source": traffic_src,
                     "reference_copy_gbs": round(copy_gbs, 1),
                     "reference_read_gbs": round(read_gbs, 1)},
        "cpu_baseline": None,
    }
    import oracle
    cores = cpu_cores()
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = wl.cpu_sample(oracle, args.cpu_seconds, cores)
        log(f"cpu oracle: {line['cpu_baseline']['value']} {line['cpu_baseline']['unit']} on {cores} threads")

    if not args.no_configs:
        t0 = time.perf_counter()
        line["allocator"] = allocator_study(pa)
        log(f"allocator study: {time.perf_counter() - t0:.1f}s")
        del wl
        torch.cuda.empty_cache()
        entries = []
        for key, over in CONFIG_SET:
            a = argparse.Namespace(**vars(args))
            a.block_size = over.get("block_size", 0)
            ps = DEFAULT_PARTITION[key]
            w = WORKLOADS[key](pa, W, torch, ps, a)
            entries.append(config_entry(key, w, torch, oracle, args, args.config_cpu_seconds, cores))
            del w
            torch.cuda.empty_cache()
        line["configs"] = entries
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
