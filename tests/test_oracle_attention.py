"""Pins for the oracle's gather + decode attention, its split/LSE path, the
cache write and the block copy.

Each pin checks the oracle against something other than itself: pure-Python
brute force (its own table walk, ``math.exp`` and loops, values decoded by
torch), torch's textbook attention routine in float64, exact special cases,
invariants of the definition, and planted mistakes that must be caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from workloads import make_decode_case, raw_view

DT = ["f32", "f16", "bf16", "fp8_e4m3"]


def torch_decode(a, dtype, scale=1.0):
    """Independent decoding path (torch casts), used only by the pins."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).double().numpy()
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a)).double().numpy()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()
    if dtype == "fp8_e4m3":
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double().numpy() * scale
    raise ValueError(dtype)


def brute_force(case, seqs=None):
    """Pure-Python decode attention: walk the table token by token."""
    q = torch_decode(case.q, case.q_dtype).tolist()
    kp = torch_decode(case.k_pool, case.kv_dtype, case.k_scale).tolist()
    vp = torch_decode(case.v_pool, case.kv_dtype, case.v_scale).tolist()
    S, H, D, bs = case.num_seqs, case.num_heads, case.head_dim, case.block_size
    G = H // case.num_kv_heads
    out = [[[0.0] * D for _ in range(H)] for _ in range(S)]
    for s in (range(S) if seqs is None else seqs):
        n = int(case.context_lens[s])
        for h in range(H):
            g = h // G
            if n == 0:
                continue
            rows = []
            for t in range(n):
                blk = int(case.block_tables[s][t // bs])
                rows.append((kp[blk][g][t % bs], vp[blk][g][t % bs]))
            sc = [case.scale * sum(q[s][h][d] * k[d] for d in range(D)) for k, _ in rows]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            tot = sum(e)
            for d in range(D):
                out[s][h][d] = sum(e[t] * rows[t][1][d] for t in range(n)) / tot
    return np.array(out)


def run_oracle(case, seqs=None):
    return oracle.paged_attention(case.q, case.q_dtype, case.k_pool, case.v_pool, case.kv_dtype,
                                  case.block_tables, case.context_lens, case.block_size,
                                  case.scale, case.k_scale, case.v_scale, seqs=seqs)


def tiny(kv_dtype="f32", H=4, Hkv=2, D=8, bs=4, ctx=(0, 1, 5, 17), q_dtype=None, salt=0, spare=7):
    q_dtype = q_dtype or ("f16" if kv_dtype == "fp8_e4m3" else kv_dtype)
    return make_decode_case("pin", "tiny", num_seqs=len(ctx), num_heads=H,
                            num_kv_heads=Hkv, head_dim=D, block_size=bs, context_lens=list(ctx),
                            kv_dtype=kv_dtype, q_dtype=q_dtype, spare_blocks=spare, append=False,
                            salt=salt + 17)


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("kv_dtype", DT)
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2), (4, 1), (6, 3)])
@pytest.mark.parametrize("bs", [1, 2, 4])
def test_matches_brute_force(kv_dtype, H, Hkv, bs):
    case = tiny(kv_dtype, H=H, Hkv=Hkv, bs=bs, ctx=(0, 1, 3, 17), salt=bs * 10 + H)
    np.testing.assert_allclose(run_oracle(case), brute_force(case), rtol=0, atol=1e-12)


def test_matches_brute_force_scaled_values():
    case = tiny("f16", H=2, Hkv=2, D=8, bs=2, ctx=(9, 4))
    case.scale = 0.731
    np.testing.assert_allclose(run_oracle(case), brute_force(case), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ textbook routine
@pytest.mark.parametrize("kv_dtype", DT)
def test_equals_contiguous_sdpa(kv_dtype):
    case = tiny(kv_dtype, H=8, Hkv=2, D=16, bs=4, ctx=(1, 7, 16, 33), salt=3)
    got = run_oracle(case)
    Q = torch_decode(case.q, case.q_dtype)
    G = case.num_heads // case.num_kv_heads
    for s, n in enumerate(case.context_lens):
        # independent gather: explicit loops over tokens
        K = np.stack([torch_decode(case.k_pool[case.block_tables[s][t // 4], :, t % 4, :],
                                   case.kv_dtype, case.k_scale) for t in range(n)])
        V = np.stack([torch_decode(case.v_pool[case.block_tables[s][t // 4], :, t % 4, :],
                                   case.kv_dtype, case.v_scale) for t in range(n)])
        q_t = torch.from_numpy(Q[s])[None, :, None, :]                         # [1,H,1,D]
        k_t = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2)[None].contiguous()
        v_t = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q_t, k_t, v_t, scale=case.scale)
        np.testing.assert_allclose(got[s], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ special cases
@pytest.mark.parametrize("kv_dtype", DT)
def test_single_token_returns_v_exactly(kv_dtype):
    case = tiny(kv_dtype, H=4, Hkv=2, ctx=(1, 1, 1), salt=5)
    got = run_oracle(case)
    G = 2
    for s in range(3):
        blk = case.block_tables[s][0]
        for h in range(4):
            v = torch_decode(case.v_pool[blk, h // G, 0, :], kv_dtype, case.v_scale)
            assert np.array_equal(got[s, h], v)


def test_identical_keys_give_mean_of_values():
    case = tiny("f32", H=2, Hkv=2, ctx=(13,), salt=6)
    s, bs = 0, case.block_size
    k0 = case.k_pool[case.block_tables[s][0], :, 0, :].copy()
    for t in range(13):
        case.k_pool[case.block_tables[s][t // bs], :, t % bs, :] = k0
    got = run_oracle(case)
    V = np.stack([case.v_pool[case.block_tables[s][t // bs], :, t % bs, :] for t in range(13)])
    np.testing.assert_allclose(got[s], V.astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)


def test_zero_scale_gives_mean_of_values():
    case = tiny("f16", H=2, Hkv=1, ctx=(11,), salt=8)
    case.scale = 0.0
    got = run_oracle(case)
    V = np.stack([case.v_pool[case.block_tables[0][t // 4], :, t % 4, :] for t in range(11)])
    np.testing.assert_allclose(got[0], np.repeat(V.astype(np.float64).mean(axis=0), 2, axis=0),
                               rtol=0, atol=1e-12)


def test_empty_context_gives_zeros():
    case = tiny("f32", ctx=(0, 0))
    assert np.array_equal(run_oracle(case), np.zeros((2, 4, 8)))


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("kv_dtype", DT)
def test_physical_placement_permutation_is_bit_identical(kv_dtype):
    case = tiny(kv_dtype, H=4, Hkv=2, ctx=(3, 9, 17), salt=9)
    base = run_oracle(case)
    perm = np.random.default_rng(0).permutation(case.num_blocks)
    k2 = np.empty_like(case.k_pool); v2 = np.empty_like(case.v_pool)
    k2[perm] = case.k_pool; v2[perm] = case.v_pool
    t2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    case.k_pool, case.v_pool, case.block_tables = k2, v2, t2.astype(np.int32)
    assert np.array_equal(run_oracle(case), base)


def test_gqa_equals_mha_with_repeated_kv():
    case = tiny("bf16", H=8, Hkv=2, ctx=(5, 12), salt=10)
    gqa = run_oracle(case)
    G = 4
    case.k_pool = np.repeat(case.k_pool, G, axis=1)
    case.v_pool = np.repeat(case.v_pool, G, axis=1)
    case.num_kv_heads = 8
    np.testing.assert_allclose(run_oracle(case), gqa, rtol=0, atol=1e-12)


def test_linear_in_values_and_shift_invariant_in_keys():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 8)); K = rng.standard_normal((19, 2, 8))
    V1 = rng.standard_normal((19, 2, 8)); V2 = rng.standard_normal((19, 2, 8))
    a, b = 0.37, -1.9
    lhs = oracle.contiguous_attention(q, K, a * V1 + b * V2, 0.3)
    rhs = a * oracle.contiguous_attention(q, K, V1, 0.3) + b * oracle.contiguous_attention(q, K, V2, 0.3)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
    u = rng.standard_normal((1, 2, 8))
    np.testing.assert_allclose(oracle.contiguous_attention(q, K + u, V1, 0.3),
                               oracle.contiguous_attention(q, K, V1, 0.3), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ split context + LSE
@pytest.mark.parametrize("P", [1, 2, 3, 5, 16, 64])
def test_partition_lse_identity(P):
    case = tiny("f16", H=4, Hkv=2, ctx=(1, 17, 40), salt=12, spare=0)
    full = run_oracle(case)
    for s, n in enumerate(case.context_lens):
        m, l, o = oracle.partition_states(case.q[s], case.q_dtype, case.k_pool, case.v_pool,
                                          case.kv_dtype, case.block_tables[s], int(n),
                                          case.block_size, case.scale, P)
        assert m.shape[1] == -(-int(n) // P)
        np.testing.assert_allclose(oracle.lse_combine(m, l, o), full[s], rtol=0, atol=1e-12)


def test_partition_states_single_partition_is_plain_softmax_stats():
    case = tiny("f32", H=2, Hkv=2, ctx=(6,), salt=13)
    m, l, o = oracle.partition_states(case.q[0], "f32", case.k_pool, case.v_pool, "f32",
                                      case.block_tables[0], 6, case.block_size, case.scale, 100)
    bf = brute_force(case)
    np.testing.assert_allclose(o[:, 0, :], bf[0], rtol=0, atol=1e-12)
    q = case.q[0].astype(np.float64)
    for h in range(2):
        z = [case.scale * float(q[h] @ case.k_pool[case.block_tables[0][t // 4], h, t % 4, :]
                                .astype(np.float64)) for t in range(6)]
        assert m[h, 0] == pytest.approx(max(z), abs=1e-12)
        assert l[h, 0] == pytest.approx(sum(math.exp(x - max(z)) for x in z), abs=1e-12)


# ------------------------------------------------------------------ planted mistakes
def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible slip in the oracle must fail at least one brute-force pin."""
    case = tiny("f32", H=4, Hkv=2, bs=2, ctx=(3, 9), salt=14)
    ref = brute_force(case)
    good = oatt._attend_one

    def wrong_group(qs, K, V, scale):          # h % Hkv instead of h // G
        H, D = qs.shape
        Hkv = K.shape[1]
        perm = [(h % Hkv) * (H // Hkv) + h // Hkv for h in range(H)]
        return good(qs[perm], K, V, scale)[np.argsort(perm)]

    mutants = {
        "no_scale": lambda qs, K, V, scale: good(qs, K, V, 1.0),
        "k_v_swapped": lambda qs, K, V, scale: good(qs, V, K, scale),
        "wrong_group": wrong_group,
        "drop_last_token": lambda qs, K, V, scale: good(qs, K[:-1], V[:-1], scale),
        "no_max_shift_sign": lambda qs, K, V, scale: good(-qs, K, V, scale),
    }
    for name, fn in mutants.items():
        monkeypatch.setattr(oatt, "_attend_one", fn)
        got = run_oracle(case)
        assert not np.allclose(got, ref, atol=1e-6), name
    monkeypatch.setattr(oatt, "_attend_one", good)

    good_gather = oatt.gather_sequence

    def off_by_one(pool, kv_dtype, row, n, bs, scale=1.0):
        t = np.arange(n)
        return oatt.decode(pool[np.asarray(row)[(t + 1) // bs], :, t % bs, :], kv_dtype, scale)
    monkeypatch.setattr(oatt, "gather_sequence", off_by_one)
    assert not np.allclose(run_oracle(case), ref, atol=1e-6)
    monkeypatch.setattr(oatt, "gather_sequence", good_gather)
    np.testing.assert_allclose(run_oracle(case), ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ cache write
@pytest.mark.parametrize("src,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                    ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3"), ("f32", "fp8_e4m3")])
def test_kv_write_by_definition(src, kv):
    case = make_decode_case("w", "tiny", num_seqs=5, num_heads=2, num_kv_heads=2, head_dim=16,
                            block_size=4, context_lens=[1, 4, 5, 8, 13], kv_dtype=kv, q_dtype=src,
                            spare_blocks=5, salt=21)
    case.slot_mapping[2] = -1                                   # a skipped token
    k0, v0 = case.k_pool.copy(), case.v_pool.copy()
    oracle.kv_write(case.k_pool, case.v_pool, kv, case.k_new, case.v_new, src,
                    case.slot_mapping, 4, case.k_scale, case.v_scale)
    touched = np.zeros(case.k_pool.shape[:1] + case.k_pool.shape[2:3], dtype=bool)
    for i, slot in enumerate(case.slot_mapping):
        if slot < 0:
            continue
        b, o = divmod(int(slot), 4)
        touched[b, o] = True
        for pool, new, sc in ((case.k_pool, case.k_new, case.k_scale), (case.v_pool, case.v_new, case.v_scale)):
            if kv == src:
                assert np.array_equal(raw_view(pool[b, :, o, :], kv), raw_view(new[i], src))
            else:   # library cast of x * float32(1/scale) after clamping
                x = torch_decode(new[i], src).astype(np.float32) * (np.float32(1) / np.float32(sc))
                ref = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                assert np.array_equal(pool[b, :, o, :], ref)
    for before, after in ((k0, case.k_pool), (v0, case.v_pool)):
        mask = np.broadcast_to(~touched[:, None, :, None], before.shape)
        assert np.array_equal(raw_view(before, kv)[mask], raw_view(after, kv)[mask])


def test_copy_blocks_by_definition():
    rng = np.random.default_rng(3)
    pools = [rng.integers(0, 2 ** 16, size=(10, 2, 4, 8), dtype=np.uint16) for _ in range(3)]
    before = [p.copy() for p in pools]
    pairs = [(1, 7), (4, 2), (9, 0)]
    oracle.copy_blocks(pools, pairs)
    for b, p in zip(before, pools):
        for src, dst in pairs:
            assert np.array_equal(p[dst], b[src])
        untouched = [i for i in range(10) if i not in (7, 2, 0)]
        assert np.array_equal(p[untouched], b[untouched])
