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
class Llama7B:
    """Llama-2-7B-shaped decode step over all 32 layers: 64 sequences at context
    4096, 32 heads x 128, block size 16, fp16 cache, 17,408-block pool per layer
    (4.25 GiB of K+V per layer, 136 GiB in all), one block table for all layers."""
    name = "llama2-7b decode step, 32 layers, fp16 KV"

    def __init__(self, pa, W, torch, partition_size):
        self.pa, self.torch = pa, torch
        self.S, self.H, self.Hkv, self.D, self.bs, self.NB, self.L = 64, 32, 32, 128, 16, 17408, 32
        self.ctx = np.full(self.S, 4096, dtype=np.int32)
        self.partition_size = partition_size
        self.layers = []
        t0 = time.time()
        for l in range(self.L):
            d = W.device_pool_case(f"llama7b_l{l}", "llama7b", num_seqs=self.S, num_heads=self.H,
                                   num_kv_heads=self.Hkv, head_dim=self.D, block_size=self.bs,
                                   context_lens=self.ctx, kv_dtype="f16", num_blocks=self.NB,
                                   layer=l, place_layer=0)
            d["out"] = torch.empty_like(d["q"])
            self.layers.append(d)
        torch.cuda.synchronize()
        log(f"generated {self.L} layers of pools in {time.time() - t0:.1f}s")
        d0 = self.layers[0]
        self.tables = torch.from_numpy(d0["tables"]).cuda()
        self.ctx_t = torch.from_numpy(self.ctx).cuda()
        self.slots = torch.from_numpy(d0["slots"]).cuda()
        ws = pa.paged_attention_workspace_size(self.S, self.H, self.D, 4096, partition_size)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda")
        self.scale = d0["scale"]
        self.attn_bytes = attention_bytes(self.ctx, self.S, self.H, self.Hkv, self.D, 2, 2, self.bs)
        self.write_bytes = write_bytes(self.S, self.Hkv, self.D, 2, 2)
        self.step_bytes = self.L * (self.attn_bytes + self.write_bytes)
        self.seq_layers_per_step = self.S * self.L

    def decode(self, l):
        d = self.layers[l]
        self.pa.paged_attention_decode(d["out"], d["q"], d["k_pool"], d["v_pool"], self.tables,
                                       self.ctx_t, max_context_len=4096, scale=self.scale,
                                       partition_size=self.partition_size, workspace=self.ws)

    def step(self):
        for l in range(self.L):
            d = self.layers[l]
            self.pa.kv_cache_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], self.slots)
            self.decode(l)

    def num_decode_units(self):
        return self.L

    def config(self):
        return {"workload": self.name, "num_seqs": self.S, "context_len": 4096, "num_layers": self.L,
                "num_heads": self.H, "num_kv_heads": self.Hkv, "head_dim": self.D,
                "block_size": self.bs, "num_blocks_per_layer": self.NB, "kv_dtype": "f16",
                "partition_size": self.partition_size}

    def cpu_sample(self, oracle, budget_s):
        """Oracle write + attention for single sequences of layer 0 (all 32 heads)."""
        torch = self.torch
        d = self.layers[0]
        nblk = 4096 // self.bs
        done, t_total = 0, 0.0
        s = 0
        while t_total < budget_s and s < self.S:
            idx = torch.from_numpy(d["tables"][s, :nblk]).long().cuda()
            kp, vp = d["k_pool"][idx].cpu().numpy(), d["v_pool"][idx].cpu().numpy()
            q = d["q"][s:s + 1].cpu().numpy()
            kn, vn = d["k_new"][s:s + 1].cpu().numpy(), d["v_new"][s:s + 1].cpu().numpy()
            table = np.arange(nblk, dtype=np.int32)[None, :]
            slot = np.array([(nblk - 1) * self.bs + self.bs - 1])
            t0 = time.perf_counter()
            oracle.kv_write(kp, vp, "f16", kn, vn, "f16", slot, self.bs)
            oracle.paged_attention(q, "f16", kp, vp, "f16", table, [4096], self.bs, self.scale)
            t_total += time.perf_counter() - t0
            done += 1
            s += 1
        return done, t_total, f"{done} sequence-layers (one sequence, all 32 heads, context 4096, layer 0)"


WORKLOADS = {"llama7b": Llama7B}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b", choices=sorted(WORKLOADS))
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU-oracle baseline sample (0 = skip)")
    ap.add_argument("--decode-iters", type=int, default=64)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_129_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload](pa, W, torch, args.partition_size)

    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        wl.step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    # dominant kernel: decode attention alone, back to back over the layers
    n = args.decode_iters
    units = wl.num_decode_units()
    start.record()
    for i in range(n):
        wl.decode(i % units)
    end.record()
    torch.cuda.synchronize()
    decode_ms = start.elapsed_time(end) / n
    achieved = wl.attn_bytes / (decode_ms * 1e-3) / 1e9
    log(f"decode attention: {decode_ms * 1e3:.1f} us per launch, {achieved:.0f} GB/s")

    value = wl.step_bytes / (ms_per_step * 1e-3) / 1e9
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
        "dtype": "f16",
        "data": "synthetic",
        "config": wl.config(),
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "decode_tokens_per_s": round(wl.seq_layers_per_step / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "paged_attention_decode",
                     "avg_launch_us": round(decode_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": wl.attn_bytes},
        "cpu_baseline": None,
    }

    if args.cpu_seconds > 0:
        import oracle
        done, secs, sample = wl.cpu_sample(oracle, args.cpu_seconds)
        line["cpu_baseline"] = {"value": round(done / secs, 3), "unit": "seq-layers/s",
                                "cores": 1, "kind": "oracle", "sample": sample,
                                "gbs_equivalent": round(done * wl.attn_bytes / wl.S / secs / 1e9, 3)}
        log(f"cpu oracle: {done} seq-layers in {secs:.1f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
