"""Cache write, block copy, gather and decode attention — plain float64 definitions.

Layout of a cache pool (one for K and one for V per layer):
``pool[block][kv_head][slot_in_block][head_dim]``; token ``t`` of a sequence
lives in ``pool[table[t // block_size], :, t % block_size, :]`` and its cache
slot number is ``table[t // block_size] * block_size + t % block_size``.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .formats import decode, e4m3_encode, int8_group_encode


# ------------------------------------------------------------------ cache write
def kv_write(k_pool: np.ndarray, v_pool: np.ndarray, kv_dtype: str,
             k_new: np.ndarray, v_new: np.ndarray, src_dtype: str,
             slot_mapping: Sequence[int], block_size: int,
             k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Store each new token's K and V once, at its slot (in place).

    One token's keys and values are computed once per step and kept for all
    later steps (KV 缓存与分页注意力 §02); a sequence's new token goes into
    the slot its block table gives it (§07).  A slot of -1 means "no token".
    Same dtype: the bytes are copied.  fp8 cache: each number is stored as
    e4m3(float32(x) * float32(1/scale)) (§11).
    """
    num_slots = k_pool.shape[0] * block_size
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= num_slots:
            continue
        b, o = divmod(int(slot), block_size)
        for pool, new, sc in ((k_pool, k_new, k_scale), (v_pool, v_new, v_scale)):
            if kv_dtype == src_dtype:
                pool[b, :, o, :] = new[i]
            elif kv_dtype == "fp8_e4m3":
                x = decode(new[i], src_dtype).astype(np.float32)      # exact widening
                inv = np.float32(1.0) / np.float32(sc)
                pool[b, :, o, :] = e4m3_encode(x * inv)
            else:
                raise ValueError(f"unsupported write {src_dtype}->{kv_dtype}")


def kv_write_int8(k_pool: np.ndarray, v_pool: np.ndarray, k_scales: np.ndarray,
                  v_scales: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, src_dtype: str,
                  slot_mapping: Sequence[int], block_size: int) -> None:
    """Cache write into an int8 cache with a scale per (token, KV head): each new
    token's head vector is quantised on its own (group-wise 8-bit integers,
    KV Cache从原理到实战 §5.2) and stored with its scale at the token's slot.
    Pools [NB, Hkv, bs, D] int8, scale pools [NB, Hkv, bs] float32."""
    num_slots = k_pool.shape[0] * block_size
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= num_slots:
            continue
        b, o = divmod(int(slot), block_size)
        for pool, scales, new in ((k_pool, k_scales, k_new), (v_pool, v_scales, v_new)):
            code, scale = int8_group_encode(decode(new[i], src_dtype).astype(np.float32))
            pool[b, :, o, :] = code
            scales[b, :, o] = scale


# ------------------------------------------------------------------ copy on write
def copy_blocks(pools: Sequence[np.ndarray], pairs: Sequence[Tuple[int, int]]) -> None:
    """Copy-on-write data copy: ``pool[dst] = pool[src]`` for every pool, pair by pair.

    Before a sequence writes into a block it shares, the block is first
    copied to a fresh one and the write goes into the copy (KV 缓存与分页注意力
    §08).  Bytes are copied unchanged.
    """
    for src, dst in pairs:
        for p in pools:
            p[dst] = p[src].copy()


def swap_blocks(dst_pools: Sequence[np.ndarray], src_pools: Sequence[np.ndarray],
                pairs: Sequence[Tuple[int, int]]) -> None:
    """Block moves between two pools (device and host): ``dst[d] = src[s]`` for every
    (s, d) pair and every pool, bytes unchanged (KV 缓存与分页注意力 §09: a
    preempted sequence's blocks go to CPU memory and come back when it resumes)."""
    for s, d in pairs:
        for dst, src in zip(dst_pools, src_pools):
            dst[d] = src[s].copy()


# ------------------------------------------------------------------ gather
def gather_sequence(pool: np.ndarray, kv_dtype: str, table_row: np.ndarray, n: int,
                    block_size: int, scale: float = 1.0) -> np.ndarray:
    """Tokens 0..n-1 of one sequence, in logical order, as float64 [n, Hkv, D].

    Logical block j of the sequence is physical block ``table_row[j]``
    (KV 缓存与分页注意力 §06–§07; Paged Attention in LLMs, "Block Table").
    Table entries past ceil(n / block_size) and slots past n are never read.
    """
    t = np.arange(n)
    blocks = np.asarray(table_row)[t // block_size]
    raw = pool[blocks, :, t % block_size, :]
    if kv_dtype == "int8":                   # scale: the [NB, Hkv, bs] pool of group scales
        return decode(raw, kv_dtype, np.asarray(scale)[blocks, :, t % block_size])
    return decode(raw, kv_dtype, scale)


# ------------------------------------------------------------------ attention
def _attend_one(qs: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """qs [H, D], K/V [n, Hkv, D] -> [H, D]; query head h reads KV head h // (H/Hkv)."""
    H, D = qs.shape
    n, Hkv, _ = K.shape
    G = H // Hkv
    qg = qs.reshape(Hkv, G, D)
    z = scale * np.einsum("kgd,nkd->kgn", qg, K)            # scores
    z = z - z.max(axis=2, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=2, keepdims=True)                     # softmax weights
    return np.einsum("kgn,nkd->kgd", w, V).reshape(H, D)     # weighted sum of values


def contiguous_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Unpaged decode attention for one sequence (float64 inputs)."""
    return _attend_one(np.asarray(q, np.float64), np.asarray(K, np.float64),
                       np.asarray(V, np.float64), scale)


def paged_attention(q: np.ndarray, q_dtype: str, k_pool: np.ndarray, v_pool: np.ndarray,
                    kv_dtype: str, block_tables: np.ndarray, context_lens: Sequence[int],
                    block_size: int, scale: float, k_scale: float = 1.0,
                    v_scale: float = 1.0, seqs: Sequence[int] = None) -> np.ndarray:
    """Decode attention over a paged cache, float64 [S, H, D].

    For each sequence: gather its keys and values through the block table,
    then out[h] = sum_t softmax_t(scale * q[h] . K[t, g(h)]) V[t, g(h)] with
    g(h) = h // (H / Hkv) (heads share KV groups: KV 缓存与分页注意力 §11;
    KV Cache从原理到实战 §5.3).  A sequence with no tokens gives zeros.
    ``seqs`` restricts the work to some sequences (others stay zero).
    """
    Q = decode(q, q_dtype)
    S, H, D = Q.shape
    out = np.zeros((S, H, D), dtype=np.float64)
    rows = range(S) if seqs is None else seqs
    for s in rows:
        n = int(context_lens[s])
        if n <= 0:
            continue
        K = gather_sequence(k_pool, kv_dtype, block_tables[s], n, block_size, k_scale)
        V = gather_sequence(v_pool, kv_dtype, block_tables[s], n, block_size, v_scale)
        out[s] = _attend_one(Q[s], K, V, scale)
    return out


# ------------------------------------------------------------------ split context
def partition_states(q: np.ndarray, q_dtype: str, k_pool: np.ndarray, v_pool: np.ndarray,
                     kv_dtype: str, table_row: np.ndarray, n: int, block_size: int,
                     scale: float, partition_size: int, k_scale: float = 1.0,
                     v_scale: float = 1.0):
    """Per-partition softmax statistics of one sequence.

    Partition p covers tokens [p*P, min((p+1)*P, n)).  For each head it returns
    the partition's largest score m_p, its sum of exp(score - m_p) l_p, and its
    own normalised output o_p.  Returns (m [H, P], l [H, P], o [H, P, D]).
    """
    Q = decode(q, q_dtype)                                    # [H, D]
    H, D = Q.shape
    K = gather_sequence(k_pool, kv_dtype, table_row, n, block_size, k_scale)
    V = gather_sequence(v_pool, kv_dtype, table_row, n, block_size, v_scale)
    Hkv = K.shape[1]
    G = H // Hkv
    P = (n + partition_size - 1) // partition_size
    m = np.zeros((H, P)); l = np.zeros((H, P)); o = np.zeros((H, P, D))
    for p in range(P):
        sl = slice(p * partition_size, min((p + 1) * partition_size, n))
        for h in range(H):
            z = scale * K[sl, h // G, :] @ Q[h]
            m[h, p] = z.max()
            e = np.exp(z - m[h, p])
            l[h, p] = e.sum()
            o[h, p] = (e @ V[sl, h // G, :]) / l[h, p]
    return m, l, o


def lse_combine(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Merge partitions: out = sum_p w_p o_p / sum_p w_p with w_p = exp(m_p - max m) l_p."""
    M = m.max(axis=-1, keepdims=True)
    w = np.exp(m - M) * l
    return (w[..., None] * o).sum(axis=-2) / w.sum(axis=-1)[..., None]
