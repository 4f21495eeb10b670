"""Pins for the oracle's multi-token (prefill / chunked prefill) attention.

Each pin checks ``oracle.prefill.paged_prefill`` against something other than
itself: a pure-Python brute force (its own table walk, ``math.exp``, values
decoded by torch); torch's own causal self-attention in float64 for whole
prompts; the defining property of chunked prefill (cutting a prompt into
chunks changes nothing: every chunk's rows equal the same rows of the
whole-prompt computation); the decode oracle for one-token chunks; placement
invariance; and planted mistakes in the row positions that must be caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import prefill as opf
from test_oracle_attention import torch_decode
from workloads import make_prefill_case


def run(case, **kw):
    return opf.paged_prefill(case.q, case.q_dtype, kw.get("k_pool", case.k_pool),
                             kw.get("v_pool", case.v_pool), case.kv_dtype,
                             kw.get("tables", case.block_tables),
                             kw.get("ctx", case.context_lens), kw.get("qs", case.query_start),
                             case.block_size, case.scale, case.k_scale, case.v_scale)


def written(case):
    """Pools after the chunk's cache write (the oracle's own write, pinned elsewhere)."""
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    oracle.kv_write(kp, vp, case.kv_dtype, case.k_new, case.v_new, case.q_dtype,
                    case.slot_mapping, case.block_size, case.k_scale, case.v_scale)
    return kp, vp


def brute_force(case, kp, vp):
    """Row by row: walk the table token by token up to the row's own position."""
    q = torch_decode(case.q, case.q_dtype).tolist()
    kd = torch_decode(kp, case.kv_dtype, case.k_scale).tolist()
    vd = torch_decode(vp, case.kv_dtype, case.v_scale).tolist()
    T, H, D, bs = case.num_tokens, case.num_heads, case.head_dim, case.block_size
    G = H // case.num_kv_heads
    out = [[[0.0] * D for _ in range(H)] for _ in range(T)]
    for s in range(case.num_seqs):
        r0, r1 = int(case.query_start[s]), int(case.query_start[s + 1])
        n = int(case.context_lens[s])
        for r in range(r0, r1):
            last = n - (r1 - r0) + (r - r0)          # this row's own position
            if last < 0:
                continue
            for h in range(H):
                g = h // G
                rows = []
                for t in range(last + 1):
                    blk = int(case.block_tables[s][t // bs])
                    rows.append((kd[blk][g][t % bs], vd[blk][g][t % bs]))
                sc = [case.scale * sum(q[r][h][d] * k[d] for d in range(D)) for k, _ in rows]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = sum(e)
                for d in range(D):
                    out[r][h][d] = sum(e[t] * rows[t][1][d] for t in range(len(rows))) / tot
    return np.array(out)


def small_case(kv="f16", H=4, Hkv=2, bs=4, prior=(0, 5, 17, 2), chunk=(3, 4, 1, 6), D=8, salt=0):
    return make_prefill_case("pin", "tiny", prior_lens=list(prior), chunk_lens=list(chunk),
                             num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                             kv_dtype=kv, q_dtype="f16" if kv == "fp8_e4m3" else kv,
                             spare_blocks=3, salt=salt)


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16", "fp8_e4m3"])
@pytest.mark.parametrize("H,Hkv,bs", [(2, 2, 1), (4, 2, 4), (3, 1, 2), (6, 2, 4)])
def test_matches_brute_force(kv, H, Hkv, bs):
    case = small_case(kv, H, Hkv, bs)
    kp, vp = written(case)
    got = run(case, k_pool=kp, v_pool=vp)
    ref = brute_force(case, kp, vp)
    assert np.abs(got - ref).max() < 1e-12


def test_rows_with_no_visible_token_are_zero():
    """A chunk longer than its context: rows before position 0 attend nothing."""
    case = small_case(prior=(0, 3), chunk=(5, 2))
    kp, vp = written(case)
    ctx = case.context_lens.copy()
    ctx[0] = 2                                   # 5 rows, 2 tokens: rows 0..2 see nothing
    got = run(case, k_pool=kp, v_pool=vp, ctx=ctx)
    assert np.all(got[0:3] == 0.0) and np.all(np.abs(got[3:5]) > 0)
    object.__setattr__(case, "context_lens", ctx)
    assert np.abs(got - brute_force(case, kp, vp)).max() < 1e-12


@pytest.mark.parametrize("kv,G", [("f32", 1), ("f16", 1), ("bf16", 4), ("f16", 3)])
def test_whole_prompt_equals_torch_causal_attention(kv, G):
    """No earlier tokens: each sequence's rows are plain causal self-attention
    over its prompt, which torch computes by its own definition (float64)."""
    Hkv = 2
    case = small_case(kv, H=G * Hkv, Hkv=Hkv, bs=4, prior=(0, 0, 0), chunk=(1, 7, 13), D=16)
    kp, vp = written(case)
    got = run(case, k_pool=kp, v_pool=vp)
    q = torch.from_numpy(torch_decode(case.q, case.q_dtype))
    kd = torch.from_numpy(torch_decode(kp, kv))
    vd = torch.from_numpy(torch_decode(vp, kv))
    for s in range(case.num_seqs):
        r0, r1 = int(case.query_start[s]), int(case.query_start[s + 1])
        n = r1 - r0
        t = torch.arange(n)
        blocks = torch.from_numpy(case.block_tables[s].astype(np.int64))[t // 4]
        K = kd[blocks, :, t % 4, :].permute(1, 0, 2).repeat_interleave(G, dim=0)   # [H, n, D]
        V = vd[blocks, :, t % 4, :].permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = q[r0:r1].permute(1, 0, 2)                                              # [H, n, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K.contiguous(), V.contiguous(), is_causal=True, scale=case.scale)
        assert np.abs(got[r0:r1] - ref.permute(1, 0, 2).numpy()).max() < 1e-12


@pytest.mark.parametrize("cuts", [(13,), (4, 9), (1, 1, 11), (5, 3, 5)])
def test_chunked_rows_equal_whole_prompt_rows(cuts):
    """Chunked prefill changes nothing: a 13-token prompt processed whole, and
    cut into chunks (each chunk seeing the tokens of the earlier ones as
    cached context), give the same row outputs."""
    H, Hkv, D, bs = 4, 2, 16, 4
    whole = make_prefill_case("pin_whole", "tiny", prior_lens=[0], chunk_lens=[13],
                              num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                              kv_dtype="f16", q_dtype="f16", spare_blocks=1)
    kp, vp = written(whole)
    ref = run(whole, k_pool=kp, v_pool=vp)
    start = 0
    for c in cuts:
        qs = np.array([0, c], dtype=np.int32)
        q_rows = whole.q[start:start + c]
        part = opf.paged_prefill(q_rows, "f16", kp, vp, "f16", whole.block_tables,
                                 [start + c], qs, bs, whole.scale)
        assert np.abs(part - ref[start:start + c]).max() < 1e-12, (cuts, start)
        start += c
    assert start == 13


def test_one_token_chunks_equal_decode():
    """A chunk of one token is a decode step: same output as the decode oracle."""
    case = small_case("bf16", H=8, Hkv=2, bs=4, prior=(0, 4, 30, 7), chunk=(1, 1, 1, 1), D=16)
    kp, vp = written(case)
    got = run(case, k_pool=kp, v_pool=vp)
    dec = oracle.paged_attention(case.q, "bf16", kp, vp, "bf16", case.block_tables,
                                 case.context_lens, case.block_size, case.scale)
    assert np.array_equal(got, dec)


def test_physical_placement_permutation_is_bit_identical():
    case = small_case("f16", prior=(9, 0, 22), chunk=(4, 5, 3))
    kp, vp = written(case)
    base = run(case, k_pool=kp, v_pool=vp)
    perm = np.random.default_rng(3).permutation(case.num_blocks)
    inv = np.argsort(perm)
    kp2, vp2 = kp[inv], vp[inv]                  # block b moves to perm[b]
    tables = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    got = run(case, k_pool=kp2, v_pool=vp2, tables=tables.astype(np.int32))
    assert np.array_equal(got, base)


def test_planted_position_mistakes_are_caught(monkeypatch):
    case = small_case("f16", prior=(6, 0, 11), chunk=(3, 5, 2))
    kp, vp = written(case)
    ref = brute_force(case, kp, vp)
    good = opf.query_positions
    mistakes = {
        "aligned to the first token": lambda n, q_len: np.arange(q_len),
        "own token not visible": lambda n, q_len: good(n, q_len) - 1,
        "one token of the future visible": lambda n, q_len: np.minimum(good(n, q_len) + 1, n - 1),
    }
    for what, fn in mistakes.items():
        monkeypatch.setattr(opf, "query_positions", fn)
        got = run(case, k_pool=kp, v_pool=vp)
        assert np.abs(got - ref).max() > 1e-3, what
    monkeypatch.setattr(opf, "query_positions", good)
    assert np.abs(run(case, k_pool=kp, v_pool=vp) - ref).max() < 1e-12
