"""GPU parity of decode attention over block tables that the library allocator
built with prefix caching: sequences admitted with token ids reuse the cached
full blocks of their common beginnings (KV 缓存与分页注意力 §11), only their own
tokens' keys and values are written (through the library's cache write), and
attention over the shared blocks must match the oracle's, which gathers the
same tables."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_129_amd as pa
from gpu_util import TOL, max_err, out_to_f64, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kv_vector(tokens, t, Hkv, D, which):
    """Keys/values of token t depend on it and everything before it: a seeded draw
    keyed by the prefix, so equal beginnings give equal cache contents."""
    seed = (hash(tuple(tokens[:t + 1])) ^ (which * 0x9E3779B9)) & 0xFFFFFFFF
    return np.random.default_rng(seed).standard_normal((Hkv, D), dtype=np.float32)


@pytest.mark.parametrize("ps", [0, 512, pa.PARTITION_BALANCED])
def test_decode_over_prefix_cached_tables(ps):
    H, Hkv, D, bs, NB = 16, 4, 128, 16, 400
    rng = np.random.default_rng(17)
    system = rng.integers(0, 50, size=200).tolist()           # a shared system prompt
    alloc = pa.BlockAllocator(NB, bs, rng.permutation(NB).astype(np.int32))
    k_pool = np.full((NB, Hkv, bs, D), np.nan, dtype=np.float16)
    v_pool = np.full((NB, Hkv, bs, D), np.nan, dtype=np.float16)
    seqs, cached_total = [], 0
    for sid in range(10):
        tail = rng.integers(0, 50, size=int(rng.integers(1, 90))).tolist()
        toks = (system[:int(rng.integers(40, 201))] if sid % 3 else system) + tail
        cached = alloc.add_seq_tokens(sid, toks)
        cached_total += cached
        tables, _ = alloc.export([sid], 64)
        for t in range(cached, len(toks)):                     # only the uncached tokens
            b, o = tables[0, t // bs], t % bs
            k_pool[b, :, o, :] = kv_vector(toks, t, Hkv, D, 1)
            v_pool[b, :, o, :] = kv_vector(toks, t, Hkv, D, 2)
        seqs.append(toks)
    assert cached_total >= 9 * 32 and alloc.stats()["prefix_hit_blocks"] > 0
    ids = list(range(10))
    tables, lens = alloc.export(ids, 64)
    say(f"[case] decode over prefix-cached tables partition={ps} reused tokens {cached_total}")
    q = rng.standard_normal((10, H, D), dtype=np.float32).astype(np.float16)
    ref = oracle.paged_attention(q, "f16", k_pool, v_pool, "f16", tables, lens, bs, 1 / np.sqrt(D))
    dq, dk, dv = to_dev(q, "f16"), to_dev(k_pool, "f16"), to_dev(v_pool, "f16")
    out = torch.full_like(dq, float("nan"))
    pa.paged_attention_decode(out, dq, dk, dv, torch.from_numpy(tables).cuda(),
                              torch.from_numpy(lens).cuda(), max_context_len=int(lens.max()),
                              scale=1 / np.sqrt(D), partition_size=ps)
    torch.cuda.synchronize()
    err = max_err(out_to_f64(out), ref, "f16")
    say(f"    max-abs error {err:.3g}")
    assert err <= TOL["f16"]
    # every sequence reads back its own keys: the shared blocks hold its prefix's values
    for sid, toks in enumerate(seqs):
        K = oracle.gather_sequence(k_pool, "f16", tables[sid], len(toks), bs)
        want = np.stack([kv_vector(toks, t, Hkv, D, 1) for t in range(len(toks))])
        assert np.array_equal(K.astype(np.float16), want.astype(np.float16))
