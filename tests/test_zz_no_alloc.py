"""The allocation-free decode entry point (static per-GPU scratch) against the
workspace entry point: same kernels and schedule, so the outputs must agree
bit for bit, and both within tolerance of the oracle.  Two calls in a row,
the second on a smaller batch, in every launch mode; a batch whose records
exceed the scratch is refused with nothing launched."""
import numpy as np
import pytest
import torch

import paged_kv_cache_129_amd as pa
import workloads as W
from gpu_util import TOL, DeviceCase, max_err, oracle_step, out_to_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cases(kind):
    if kind == "gqa_bf16":
        big = W.make_decode_case("noalloc_gqa_big", "tiny", num_seqs=40, num_heads=64,
                                 num_kv_heads=8, head_dim=128, block_size=16,
                                 context_lens=W.llama70b_independent_lengths(40)[:40],
                                 kv_dtype="bf16", q_dtype="bf16", spare_blocks=16)
        small = W.make_decode_case("noalloc_gqa_small", "tiny", num_seqs=7, num_heads=64,
                                   num_kv_heads=8, head_dim=128, block_size=16,
                                   context_lens=[1, 16, 17, 600, 0, 2000, 33],
                                   kv_dtype="bf16", q_dtype="bf16", spare_blocks=16)
    elif kind == "mqa_fp8":
        big = W.make_decode_case("noalloc_mqa_big", "falcon7b", num_seqs=64, num_heads=71,
                                 num_kv_heads=1, head_dim=64, block_size=16,
                                 context_lens=W.falcon7b_lengths(64), kv_dtype="fp8_e4m3",
                                 q_dtype="f16", spare_blocks=16)
        small = W.make_decode_case("noalloc_mqa_small", "falcon7b", num_seqs=5, num_heads=71,
                                   num_kv_heads=1, head_dim=64, block_size=16,
                                   context_lens=[3, 512, 513, 1000, 1], kv_dtype="fp8_e4m3",
                                   q_dtype="f16", spare_blocks=16)
    else:
        big = W.make_decode_case("noalloc_mha_big", "opt13b", num_seqs=24, num_heads=40,
                                 num_kv_heads=40, head_dim=128, block_size=16,
                                 context_lens=np.linspace(1, 1800, 24).astype(int),
                                 kv_dtype="f16", q_dtype="f16", spare_blocks=16)
        small = W.make_decode_case("noalloc_mha_small", "opt13b", num_seqs=3, num_heads=40,
                                   num_kv_heads=40, head_dim=128, block_size=16,
                                   context_lens=[700, 5, 64], kv_dtype="f16", q_dtype="f16",
                                   spare_blocks=16)
    return big, small


@pytest.mark.parametrize("ps", [0, 512, pa.PARTITION_BALANCED])
@pytest.mark.parametrize("kind", ["gqa_bf16", "mqa_fp8", "mha_f16"])
def test_noalloc_matches_workspace_entry_point(kind, ps):
    for case in _cases(kind):
        say(f"[case] noalloc {case.name} partition={ps} S={case.num_seqs}")
        _, _, ref = oracle_step(case)
        dev = DeviceCase(case)
        dev.write()
        want = dev.attend(ps, out=torch.full_like(dev.q, float("nan")))
        got = torch.full_like(dev.q, float("nan"))
        pa.paged_attention_decode_noalloc(got, dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.ctx,
                                          max_context_len=case.max_context_len, scale=case.scale,
                                          k_scale=case.k_scale, v_scale=case.v_scale,
                                          partition_size=ps)
        torch.cuda.synchronize()
        g, w = out_to_f64(got), out_to_f64(want)
        assert np.array_equal(g, w), (case.name, ps, float(np.abs(g - w).max()))
        err = max_err(g, ref, case.q_dtype)
        say(f"    max-abs error vs oracle {err:.3g}")
        assert err <= TOL[case.kv_dtype]


def test_noalloc_refuses_records_beyond_scratch():
    """Partitions of 16 tokens over 2,048 sequences x 64 heads x 128 need
    2048*64*256*130*4 bytes of records, far beyond the scratch: refused."""
    S, H, Hkv, D = 2048, 64, 8, 128
    q = torch.zeros(S, H, D, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(8, Hkv, 16, D, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(S, 256, dtype=torch.int32, device="cuda")
    ctx = torch.ones(S, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pa.PagedAttnError, match="PA_ERR_WORKSPACE"):
        pa.paged_attention_decode_noalloc(out, q, pool, pool, tables, ctx, max_context_len=4096,
                                          scale=0.1, partition_size=16)
