"""Seeded synthetic inputs for paged decode attention.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and lays them out: context lengths,
physical block placement (a seeded shuffle of the pool), q/K/V values stored
in the cache dtype, and NaN poison for every slot that no sequence owns.  It
holds none of the method's arithmetic (no attention, no cache write, no
quantisation code of its own: the one fp8 cast used for pre-existing cache
contents is torch's library cast).

Pool layout (one pool for K and one for V, per layer):
    pool[block][kv_head][slot_in_block][head_dim]
so that one (block, kv-head) tile is a dense ``block_size x head_dim`` array.
``slot = physical_block * block_size + offset`` addresses one token.

Recipes follow the workload shapes of the pages (KV 缓存与分页注意力 §03, §06,
§11; KV Cache从原理到实战 §2.2): OPT-13B-, Llama-2-7B-, Llama-2-70B- and
Falcon-7B-shaped layers with synthetic N(0,1) values; no dataset or weights.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------- dtypes
DTYPES = ("f32", "f16", "bf16", "fp8_e4m3")
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8,
           "int8": np.int8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1, "int8": 1}
# quiet-NaN bit patterns used to poison slots that hold no live token (int8
# codes: -128, which the group-wise codec never writes; its scale slots hold NaN)
POISON_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F, "int8": 0x80}
_RAW = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8_e4m3": np.uint8,
        "int8": np.uint8}


def raw_view(a: np.ndarray, dtype: str) -> np.ndarray:
    """Bit view of a storage array (for bit-exact comparisons)."""
    return a.view(_RAW[dtype])


def poison_value(dtype: str):
    return np.array([POISON_BITS[dtype]], dtype=_RAW[dtype]).view(STORAGE[dtype])[0]


def empty_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
               dtype: str) -> np.ndarray:
    pool = np.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=STORAGE[dtype])
    raw_view(pool, dtype)[...] = POISON_BITS[dtype]
    return pool


# ---------------------------------------------------------------- seeds
_CONFIG_IDS = {"tiny": 1, "opt13b": 2, "llama7b": 3, "llama70b": 4, "falcon7b": 5}
_TENSOR_IDS = {"ctx": 0, "place": 1, "q": 2, "k": 3, "v": 4, "knew": 5, "vnew": 6,
               "group": 7, "prompt_k": 8, "prompt_v": 9, "free": 10, "misc": 11}


def rng_for(config: str, layer: int, tensor: str, salt: int = 0) -> np.random.Generator:
    """One independent stream per (config, layer, tensor); base seed 0."""
    key = (_CONFIG_IDS.get(config, 99), layer, _TENSOR_IDS[tensor], salt)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(0, spawn_key=key)))


# ---------------------------------------------------------------- storage casts
def to_storage(x: np.ndarray, dtype: str, scale: Optional[float] = None) -> np.ndarray:
    """Round fp32 values into the storage dtype (RNE).

    fp8 values are ``x * float32(1/scale)`` cast by torch's e4m3fn cast after
    clamping to the format's finite range; this only produces pre-existing
    cache contents, both implementations under test read the same bytes.
    """
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16)
    import torch
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8_e4m3":
        assert scale is not None and scale > 0
        inv = np.float32(1.0) / np.float32(scale)
        y = torch.from_numpy(x * inv).clamp(-448.0, 448.0)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening used only to compute calibration scales (amax)."""
    if dtype in ("f32", "f16"):
        return a.astype(np.float32)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------- lengths, placement
def lognormal_lengths(rng: np.random.Generator, n: int, median: float, lo: int, hi: int,
                      sigma: float = 0.8) -> np.ndarray:
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def uniform_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


def blocks_needed(ctx: Sequence[int], block_size: int) -> np.ndarray:
    c = np.asarray(ctx, dtype=np.int64)
    return (c + block_size - 1) // block_size


def place_blocks(rng: np.random.Generator, num_blocks: int, nblocks_per_seq: Sequence[int],
                 max_blocks: Optional[int] = None) -> np.ndarray:
    """Random distinct physical blocks for each sequence (seeded shuffle of the pool).

    Returns int32 tables [S, max_blocks], padded with -1.
    """
    nb = np.asarray(nblocks_per_seq, dtype=np.int64)
    total = int(nb.sum())
    if total > num_blocks:
        raise ValueError(f"need {total} blocks, pool has {num_blocks}")
    mb = int(max(1, nb.max(initial=0))) if max_blocks is None else max_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(nb), mb), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(nb):
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    return tables


def slots_of(tables: np.ndarray, positions: Sequence[int], block_size: int) -> np.ndarray:
    """slot = physical_block * block_size + offset for token ``positions[s]`` of row s."""
    pos = np.asarray(positions, dtype=np.int64)
    out = np.full(len(pos), -1, dtype=np.int64)
    for s, p in enumerate(pos):
        if p >= 0:
            out[s] = int(tables[s, p // block_size]) * block_size + int(p % block_size)
    return out


def fill_tokens(pool: np.ndarray, table_row: np.ndarray, values: np.ndarray, block_size: int,
                start: int = 0) -> None:
    """Store ``values[i]`` ([Hkv, D]) as token ``start + i`` of a sequence."""
    n = values.shape[0]
    if n == 0:
        return
    t = np.arange(start, start + n)
    blocks = table_row[t // block_size]
    offs = t % block_size
    pool[blocks, :, offs, :] = values


# ---------------------------------------------------------------- one decode case
@dataclasses.dataclass
class DecodeCase:
    """One layer's decode step: pre-append pools, the new token, and the query.

    ``context_lens`` count the new token (it sits at position ctx-1 and is
    written by the cache-write call before attention reads it).
    """
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str
    q_dtype: str
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, MB], -1 padded
    k_pool: np.ndarray                # storage [NB, Hkv, bs, D]  (pre-append)
    v_pool: np.ndarray
    k_new: np.ndarray                 # q_dtype storage [S, Hkv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray          # int64 [S]; -1 = no new token
    q: np.ndarray                     # q_dtype storage [S, H, D]
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    partition_size: int = 0
    k_scales: Optional[np.ndarray] = None   # int8 cache: float32 [NB, Hkv, bs] (pre-append)
    v_scales: Optional[np.ndarray] = None

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max(initial=0))


def make_decode_case(name: str, config: str, *, num_seqs: int, num_heads: int, num_kv_heads: int,
                     head_dim: int, block_size: int, context_lens: Sequence[int],
                     kv_dtype: str, q_dtype: str, num_blocks: Optional[int] = None,
                     value_scale: float = 1.0, layer: int = 0, partition_size: int = 0,
                     spare_blocks: int = 0, append: bool = True, salt: int = 0,
                     max_blocks: Optional[int] = None, key_drift: Optional[str] = None) -> DecodeCase:
    """Build one case: shuffled placement, N(0,1)*value_scale values, poison elsewhere.

    ``key_drift`` adds a position-dependent amount c(t) to the first head_dim
    component of every key, and 3.0 to that component of every query, so the
    scores follow c: "rising" (c = t / 2), "falling" (c = (n - 1 - t) / 2 for a
    context of n), or "spikes" (c = 12..24 at every 29th position, else 0)."""
    ctx = np.asarray(context_lens, dtype=np.int32)
    S, H, Hkv, D, bs = num_seqs, num_heads, num_kv_heads, head_dim, block_size
    assert ctx.shape == (S,) and H % Hkv == 0
    nbs = blocks_needed(ctx, bs)
    NB = int(nbs.sum()) + spare_blocks if num_blocks is None else num_blocks
    tables = place_blocks(rng_for(config, layer, "place", salt), NB, nbs, max_blocks)

    # fp32 draws: pre-existing tokens, the new token, the query
    pre = np.maximum(ctx - (1 if append else 0), 0)
    rk, rv = rng_for(config, layer, "k", salt), rng_for(config, layer, "v", salt)
    k_vals = [(rk.standard_normal((int(n), Hkv, D), dtype=np.float32) * np.float32(value_scale))
              for n in pre]
    v_vals = [(rv.standard_normal((int(n), Hkv, D), dtype=np.float32) * np.float32(value_scale))
              for n in pre]
    src_dtype = q_dtype
    k_new32 = rng_for(config, layer, "knew", salt).standard_normal((S, Hkv, D), dtype=np.float32) \
        * np.float32(value_scale)
    q32 = rng_for(config, layer, "q", salt).standard_normal((S, H, D), dtype=np.float32) \
        * np.float32(value_scale)
    if key_drift is not None:
        def drift(t: np.ndarray, n: int) -> np.ndarray:
            if key_drift == "rising":
                return 0.5 * t
            if key_drift == "falling":
                return 0.5 * (n - 1 - t)
            if key_drift == "spikes":
                return np.where(t % 29 == 7, 12.0 + 3.0 * ((t // 29) % 5), 0.0)
            raise ValueError(key_drift)
        for s in range(S):
            n = int(pre[s])
            k_vals[s][:, :, 0] += drift(np.arange(n), int(ctx[s]))[:, None].astype(np.float32)
            if ctx[s] > 0:
                k_new32[s, :, 0] += np.float32(drift(np.array([int(ctx[s]) - 1]), int(ctx[s]))[0])
        q32[:, :, 0] += np.float32(3.0)
    v_new32 = rng_for(config, layer, "vnew", salt).standard_normal((S, Hkv, D), dtype=np.float32) \
        * np.float32(value_scale)
    k_new = to_storage(k_new32, src_dtype)
    v_new = to_storage(v_new32, src_dtype)
    q = to_storage(q32, q_dtype)

    k_scale = v_scale = 1.0
    if kv_dtype == "fp8_e4m3":
        # per-tensor calibration: scale = amax / 448 over everything stored in the tensor
        def amax(vals, new):
            m = float(np.abs(storage_to_f32(new, src_dtype)).max(initial=0.0))
            for a in vals:
                if a.size:
                    m = max(m, float(np.abs(a).max()))
            return m
        k_scale = float(np.float32(max(amax(k_vals, k_new), 1e-30) / 448.0))
        v_scale = float(np.float32(max(amax(v_vals, v_new), 1e-30) / 448.0))

    k_pool = empty_pool(NB, Hkv, bs, D, kv_dtype)
    v_pool = empty_pool(NB, Hkv, bs, D, kv_dtype)
    for s in range(S):
        fill_tokens(k_pool, tables[s], to_storage(k_vals[s], kv_dtype, k_scale), bs)
        fill_tokens(v_pool, tables[s], to_storage(v_vals[s], kv_dtype, v_scale), bs)
    if append:
        slot_mapping = slots_of(tables, ctx.astype(np.int64) - 1, bs)
    else:
        slot_mapping = np.full(S, -1, dtype=np.int64)
    return DecodeCase(name=name, num_seqs=S, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                      block_size=bs, num_blocks=NB, kv_dtype=kv_dtype, q_dtype=q_dtype,
                      context_lens=ctx, block_tables=tables, k_pool=k_pool, v_pool=v_pool,
                      k_new=k_new, v_new=v_new, slot_mapping=slot_mapping, q=q,
                      scale=1.0 / math.sqrt(D), k_scale=k_scale, v_scale=v_scale,
                      partition_size=partition_size)


def int8_storage(x: np.ndarray):
    """Pre-existing contents of a group-wise int8 cache: fp32 head vectors
    [..., D] -> (int8 codes, float32 scales [...]), one scale per vector set to
    its amax / 127 and the codes made by torch's per-channel int8 quantiser
    with those scales.  Like the fp8 cast above this only lays out inputs:
    both implementations under test read the same bytes and scales."""
    import torch
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1, x.shape[-1])
    if flat.shape[0] == 0:
        return np.zeros(x.shape, np.int8), np.zeros(x.shape[:-1], np.float32)
    amax = np.abs(flat).max(axis=1)
    sc = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(sc > 0, sc, np.float32(1)).astype(np.float64)
    tq = torch.quantize_per_channel(torch.from_numpy(flat), torch.from_numpy(safe),
                                    torch.zeros(len(flat), dtype=torch.int64), 0, torch.qint8)
    codes = np.maximum(tq.int_repr().numpy(), -127).astype(np.int8)
    return codes.reshape(x.shape), sc.reshape(x.shape[:-1])


def make_int8_case(name: str, config: str, *, num_seqs: int, num_heads: int, num_kv_heads: int,
                   head_dim: int, block_size: int, context_lens: Sequence[int], q_dtype: str,
                   num_blocks: Optional[int] = None, spare_blocks: int = 0, salt: int = 0,
                   value_scale: float = 1.0) -> DecodeCase:
    """A decode case over a group-wise int8 cache: the placement, lengths and
    N(0,1) * value_scale draws of make_decode_case, pre-existing tokens stored as
    int8 codes with a float32 scale per (token, KV head) (int8_storage); unused
    slots hold code -128 and a NaN scale.  The new token's K/V stay in q_dtype
    for the quantising cache write."""
    base = make_decode_case(name, config, num_seqs=num_seqs, num_heads=num_heads,
                            num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                            context_lens=context_lens, kv_dtype="f32", q_dtype=q_dtype,
                            num_blocks=num_blocks, spare_blocks=spare_blocks, salt=salt,
                            value_scale=value_scale)
    NB, Hkv, bs, D = base.k_pool.shape
    pools, scales = [], []
    for src in (base.k_pool, base.v_pool):
        pool = empty_pool(NB, Hkv, bs, D, "int8")
        sc = np.full((NB, Hkv, bs), np.nan, dtype=np.float32)
        live = ~np.isnan(src).any(axis=-1)              # slots holding a pre-existing token
        codes, s = int8_storage(src[live])
        pool[live] = codes
        sc[live] = s
        pools.append(pool)
        scales.append(sc)
    return dataclasses.replace(base, kv_dtype="int8", k_pool=pools[0], v_pool=pools[1],
                               k_scales=scales[0], v_scales=scales[1])


# ---------------------------------------------------------------- the five workloads
def tiny_case(salt: int = 0) -> DecodeCase:
    """1 layer, 4 sequences, ctx {5,10,3,16}, 2 heads, D 64, bs 4, 44 blocks, fp32."""
    return make_decode_case("tiny_fp32", "tiny", num_seqs=4, num_heads=2, num_kv_heads=2,
                            head_dim=64, block_size=4, context_lens=[5, 10, 3, 16],
                            kv_dtype="f32", q_dtype="f32", num_blocks=44, salt=salt)


def opt13b_lengths(n: int = 30, num_blocks: int = 1000, block_size: int = 16):
    """Log-normal lengths (median 300, sigma 0.8, clip 1..2048); redraw until they fit."""
    for salt in range(1000):
        ctx = lognormal_lengths(rng_for("opt13b", 0, "ctx", salt), n, 300, 1, 2048)
        if int(blocks_needed(ctx, block_size).sum()) <= num_blocks:
            return ctx, salt
    raise RuntimeError("no fitting draw")


def opt13b_case(num_seqs: int = 30) -> DecodeCase:
    ctx, _ = opt13b_lengths(num_seqs)
    return make_decode_case("opt13b_fp16", "opt13b", num_seqs=num_seqs, num_heads=40,
                            num_kv_heads=40, head_dim=128, block_size=16, context_lens=ctx,
                            kv_dtype="f16", q_dtype="f16", num_blocks=1000,
                            value_scale=1.0 / math.sqrt(128))


def falcon7b_lengths(n: int = 256) -> np.ndarray:
    return uniform_lengths(rng_for("falcon7b", 0, "ctx"), n, 1, 2048)


def falcon7b_num_blocks(ctx: Sequence[int], block_size: int) -> int:
    return int(math.ceil(1.25 * int(blocks_needed(ctx, block_size).sum())))


def llama70b_independent_lengths(n: int = 96) -> np.ndarray:
    return lognormal_lengths(rng_for("llama70b", 0, "ctx"), n, 1024, 128, 8192)


@dataclasses.dataclass
class SharedPromptSpec:
    """Llama-2-70B-shaped GQA batch: independent sequences plus parallel-sample groups.

    ``prompt_len`` tokens are shared by ``samples`` sequences of each group; the
    first append of every sample after the fork lands in the shared,
    partially filled last prompt block.
    """
    independent_ctx: np.ndarray      # pre-append lengths of independent sequences
    groups: int
    samples: int
    prompt_len: int


def llama70b_spec(independent: int = 96, groups: int = 8, samples: int = 4,
                  prompt_len: int = 520) -> SharedPromptSpec:
    ctx = llama70b_independent_lengths(independent) - 1   # pre-append
    return SharedPromptSpec(independent_ctx=ctx.astype(np.int32), groups=groups, samples=samples,
                            prompt_len=prompt_len)


def token_values(config: str, tensor: str, stream: int, n: int, num_kv_heads: int,
                 head_dim: int, value_scale: float = 1.0, layer: int = 0) -> np.ndarray:
    """fp32 N(0,1) values for ``n`` tokens of stream ``stream`` (a sequence or a prompt)."""
    r = rng_for(config, layer, tensor, salt=stream)
    return r.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32) * np.float32(value_scale)


def shared_prompt_case(alloc, spec: SharedPromptSpec, *, num_heads: int = 64, num_kv_heads: int = 8,
                       head_dim: int = 128, block_size: int = 16, num_blocks: int = 12288,
                       kv_dtype: str = "bf16", q_dtype: str = "bf16", config: str = "llama70b",
                       layer: int = 0):
    """Parallel-sampling batch laid out by ``alloc`` (any object with add_seq / fork /
    append_slots / export, e.g. the library allocator or the oracle's model).

    Independent sequences get their own blocks; each group's ``samples``
    sequences fork one prompt and so share its blocks.  The pool holds the
    pre-append tokens (values drawn per sequence / per prompt); the returned
    case carries the post-append tables and lengths, the slots of the new
    tokens, and the copy-on-write pairs the allocator emitted, which must be
    applied before the write.
    """
    ctx_pre = np.asarray(spec.independent_ctx, dtype=np.int64)
    n_ind = len(ctx_pre)
    S = n_ind + spec.groups * spec.samples
    H, Hkv, D, bs = num_heads, num_kv_heads, head_dim, block_size
    for i, n in enumerate(ctx_pre):
        alloc.add_seq(i, int(n))
    for g in range(spec.groups):
        parent = n_ind + g * spec.samples
        alloc.add_seq(parent, spec.prompt_len)
        for j in range(1, spec.samples):
            alloc.fork(parent, parent + j)
    ids = list(range(S))
    pre_lens = np.concatenate([ctx_pre, np.full(spec.groups * spec.samples, spec.prompt_len)])
    max_blocks = int((int(pre_lens.max()) + 1 + bs - 1) // bs) + 1
    tables_pre, lens_pre = alloc.export(ids, max_blocks)
    k_pool = empty_pool(num_blocks, Hkv, bs, D, kv_dtype)
    v_pool = empty_pool(num_blocks, Hkv, bs, D, kv_dtype)
    for i in range(n_ind):
        n = int(ctx_pre[i])
        fill_tokens(k_pool, tables_pre[i], to_storage(token_values(config, "k", i, n, Hkv, D,
                                                                   layer=layer), kv_dtype), bs)
        fill_tokens(v_pool, tables_pre[i], to_storage(token_values(config, "v", i, n, Hkv, D,
                                                                   layer=layer), kv_dtype), bs)
    for g in range(spec.groups):
        parent = n_ind + g * spec.samples
        P = spec.prompt_len
        fill_tokens(k_pool, tables_pre[parent], to_storage(
            token_values(config, "prompt_k", g, P, Hkv, D, layer=layer), kv_dtype), bs)
        fill_tokens(v_pool, tables_pre[parent], to_storage(
            token_values(config, "prompt_v", g, P, Hkv, D, layer=layer), kv_dtype), bs)
    slots, pairs = alloc.append_slots(ids)
    tables, lens = alloc.export(ids, max_blocks)
    r = rng_for(config, layer, "misc")
    k_new = to_storage(r.standard_normal((S, Hkv, D), dtype=np.float32), q_dtype)
    v_new = to_storage(r.standard_normal((S, Hkv, D), dtype=np.float32), q_dtype)
    q = to_storage(r.standard_normal((S, H, D), dtype=np.float32), q_dtype)
    case = DecodeCase(name=f"{config}_shared", num_seqs=S, num_heads=H, num_kv_heads=Hkv,
                      head_dim=D, block_size=bs, num_blocks=num_blocks, kv_dtype=kv_dtype,
                      q_dtype=q_dtype, context_lens=np.asarray(lens, dtype=np.int32),
                      block_tables=np.asarray(tables, dtype=np.int32), k_pool=k_pool,
                      v_pool=v_pool, k_new=k_new, v_new=v_new,
                      slot_mapping=np.asarray(slots, dtype=np.int64), q=q,
                      scale=1.0 / math.sqrt(D))
    return case, np.asarray(pairs, dtype=np.int32).reshape(-1, 2)


def free_order(config: str, num_blocks: int) -> np.ndarray:
    """Seeded shuffle of the pool used as an allocator's initial free list."""
    return rng_for(config, 0, "free").permutation(num_blocks).astype(np.int32)


def device_pool_case(name: str, config: str, *, num_seqs: int, num_heads: int, num_kv_heads: int,
                     head_dim: int, block_size: int, context_lens: Sequence[int], kv_dtype: str,
                     num_blocks: int, layer: int = 0, device: str = "cuda", seed: int = 0,
                     max_blocks: Optional[int] = None, place_layer: Optional[int] = None):
    """Large decode case generated on the device with torch's seeded generator.

    Returns a dict of device tensors (pre-append pools with NaN poison in
    every slot that holds no live token, new tokens, query, tables, lengths,
    slots).  Used where host generation would be too slow (4 GiB pools).
    """
    import torch
    ctx = np.asarray(context_lens, dtype=np.int32)
    S, H, Hkv, D, bs = num_seqs, num_heads, num_kv_heads, head_dim, block_size
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[kv_dtype]
    nbs = blocks_needed(ctx, bs)
    # one block table per sequence serves every layer: placement may come from another layer
    tables = place_blocks(rng_for(config, layer if place_layer is None else place_layer, "place"),
                          num_blocks, nbs, max_blocks)
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (layer + 1) + 7919 * seed + _CONFIG_IDS.get(config, 99))
    shape = (num_blocks, Hkv, bs, D)
    k_pool = torch.empty(shape, dtype=tdt, device=device)
    v_pool = torch.empty(shape, dtype=tdt, device=device)
    for p in (k_pool, v_pool):
        for b0 in range(0, num_blocks, 4096):          # bounded temporaries
            b1 = min(num_blocks, b0 + 4096)
            p[b0:b1].normal_(generator=g)
    nan = float("nan")
    used = np.zeros(num_blocks, dtype=bool)
    for s in range(S):
        used[tables[s, :nbs[s]]] = True
    free = torch.from_numpy(np.nonzero(~used)[0]).to(device)
    for p in (k_pool, v_pool):
        if free.numel():
            p[free] = nan
        for s in range(S):
            n = int(ctx[s])
            for t in range(max(n - 1, 0), int(nbs[s]) * bs):       # new token's slot and the tail
                p[int(tables[s, t // bs]), :, t % bs, :] = nan
    k_new = torch.randn((S, Hkv, D), generator=g, device=device, dtype=torch.float32).to(tdt)
    v_new = torch.randn((S, Hkv, D), generator=g, device=device, dtype=torch.float32).to(tdt)
    q = torch.randn((S, H, D), generator=g, device=device, dtype=torch.float32).to(tdt)
    slots = slots_of(tables, ctx.astype(np.int64) - 1, bs)
    return dict(name=name, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, q=q,
                tables=tables, ctx=ctx, slots=slots, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                block_size=bs, num_blocks=num_blocks, kv_dtype=kv_dtype, scale=1.0 / math.sqrt(D))


# ---------------------------------------------------------------- multi-token (prefill) cases
@dataclasses.dataclass
class PrefillCase:
    """One layer's chunked-prefill step: pools holding each sequence's earlier
    tokens, the chunk's new K/V (written through their slots before attention)
    and the chunk's queries, packed row after row.

    ``context_lens`` count the chunk; sequence s's query rows are
    ``query_start[s]:query_start[s+1]`` and belong to its last
    ``query_start[s+1] - query_start[s]`` positions.
    """
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str
    q_dtype: str
    context_lens: np.ndarray          # int32 [S], chunk included
    query_start: np.ndarray           # int32 [S + 1]
    block_tables: np.ndarray          # int32 [S, MB], -1 padded
    k_pool: np.ndarray                # storage [NB, Hkv, bs, D] (before the chunk's write)
    v_pool: np.ndarray
    k_new: np.ndarray                 # q_dtype storage [T, Hkv, D]
    v_new: np.ndarray
    slot_mapping: np.ndarray          # int64 [T]
    q: np.ndarray                     # q_dtype storage [T, H, D]
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])

    @property
    def max_query_len(self) -> int:
        return int(np.diff(self.query_start).max(initial=0))

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max(initial=0))


def make_prefill_case(name: str, config: str, *, prior_lens: Sequence[int],
                      chunk_lens: Sequence[int], num_heads: int, num_kv_heads: int,
                      head_dim: int, block_size: int, kv_dtype: str, q_dtype: str,
                      num_blocks: Optional[int] = None, spare_blocks: int = 0,
                      value_scale: float = 1.0, layer: int = 0, salt: int = 0) -> PrefillCase:
    """Sequences with ``prior_lens[s]`` tokens already cached and a chunk of
    ``chunk_lens[s]`` new tokens; shuffled placement, N(0,1)*value_scale values,
    NaN poison in every slot no earlier token owns (the chunk's slots included,
    until the write)."""
    prior = np.asarray(prior_lens, dtype=np.int64)
    chunk = np.asarray(chunk_lens, dtype=np.int64)
    S, H, Hkv, D, bs = len(prior), num_heads, num_kv_heads, head_dim, block_size
    assert chunk.shape == (S,) and H % Hkv == 0
    ctx = (prior + chunk).astype(np.int32)
    nbs = blocks_needed(ctx, bs)
    NB = int(nbs.sum()) + spare_blocks if num_blocks is None else num_blocks
    tables = place_blocks(rng_for(config, layer, "place", 100 + salt), NB, nbs)
    rk, rv = rng_for(config, layer, "k", 100 + salt), rng_for(config, layer, "v", 100 + salt)
    k_vals = [rk.standard_normal((int(n), Hkv, D), dtype=np.float32) * np.float32(value_scale)
              for n in prior]
    v_vals = [rv.standard_normal((int(n), Hkv, D), dtype=np.float32) * np.float32(value_scale)
              for n in prior]
    T = int(chunk.sum())
    k_new32 = rng_for(config, layer, "knew", 100 + salt).standard_normal((T, Hkv, D), dtype=np.float32) \
        * np.float32(value_scale)
    v_new32 = rng_for(config, layer, "vnew", 100 + salt).standard_normal((T, Hkv, D), dtype=np.float32) \
        * np.float32(value_scale)
    q32 = rng_for(config, layer, "q", 100 + salt).standard_normal((T, H, D), dtype=np.float32) \
        * np.float32(value_scale)
    k_new, v_new, q = (to_storage(x, q_dtype) for x in (k_new32, v_new32, q32))
    k_scale = v_scale = 1.0
    if kv_dtype == "fp8_e4m3":
        def amax(vals, new):
            m = float(np.abs(storage_to_f32(new, q_dtype)).max(initial=0.0))
            for a in vals:
                if a.size:
                    m = max(m, float(np.abs(a).max()))
            return m
        k_scale = float(np.float32(max(amax(k_vals, k_new), 1e-30) / 448.0))
        v_scale = float(np.float32(max(amax(v_vals, v_new), 1e-30) / 448.0))
    k_pool = empty_pool(NB, Hkv, bs, D, kv_dtype)
    v_pool = empty_pool(NB, Hkv, bs, D, kv_dtype)
    for s in range(S):
        fill_tokens(k_pool, tables[s], to_storage(k_vals[s], kv_dtype, k_scale), bs)
        fill_tokens(v_pool, tables[s], to_storage(v_vals[s], kv_dtype, v_scale), bs)
    query_start = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    slots = np.empty(T, dtype=np.int64)
    for s in range(S):
        pos = prior[s] + np.arange(chunk[s])
        slots[query_start[s]:query_start[s + 1]] = \
            tables[s, pos // bs].astype(np.int64) * bs + pos % bs
    return PrefillCase(name=name, num_seqs=S, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                       block_size=bs, num_blocks=NB, kv_dtype=kv_dtype, q_dtype=q_dtype,
                       context_lens=ctx, query_start=query_start, block_tables=tables,
                       k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
                       slot_mapping=slots, q=q, scale=1.0 / math.sqrt(D), k_scale=k_scale,
                       v_scale=v_scale)


def llama7b_prefill_case(num_seqs: int = 8, chunk: int = 512, layer: int = 0) -> PrefillCase:
    """Llama-2-7B-shaped chunked prefill: 32 heads x 128, fp16, block 16; sequence s
    has s * 512 tokens cached and a 512-token chunk, so contexts run 512..4096."""
    prior = [chunk * s for s in range(num_seqs)]
    return make_prefill_case("llama7b_prefill", "llama7b", prior_lens=prior,
                             chunk_lens=[chunk] * num_seqs, num_heads=32, num_kv_heads=32,
                             head_dim=128, block_size=16, kv_dtype="f16", q_dtype="f16",
                             spare_blocks=64, layer=layer)
