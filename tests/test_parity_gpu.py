"""GPU parity: the library (through the C ABI) against the oracle on the same
seeded inputs.  Cache writes and block copies must be bit-exact; attention
must be within max-abs 1e-4 (fp32 cache), 5e-3 (fp16/bf16) or 3e-2 (fp8,
where the oracle dequantises the same stored codes)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_129_amd as pa
import workloads as W
from gpu_util import (TOL, DeviceCase, assert_pools_equal, from_dev, max_err, oracle_step,
                      out_to_f64, raw_err, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"device: {torch.cuda.get_device_name(0)}; {pa.version()}")


def run_and_check(case, partitions=(0,), label=""):
    say(f"[case] {case.name} {label} S={case.num_seqs} H={case.num_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} bs={case.block_size} kv={case.kv_dtype} q={case.q_dtype} "
        f"max_ctx={case.max_context_len} parts={partitions}")
    kp, vp, ref = oracle_step(case)
    dev = DeviceCase(case)
    dev.write()
    torch.cuda.synchronize()
    assert_pools_equal(dev, kp, vp)
    errs, raws = {}, {}
    for ps in partitions:
        out = dev.attend(ps, out=torch.full_like(dev.q, float("nan")))   # every element written
        torch.cuda.synchronize()
        got = out_to_f64(out)
        errs[ps] = max_err(got, ref, case.q_dtype)
        raws[ps] = raw_err(got, ref)
        assert errs[ps] <= TOL[case.kv_dtype], (case.name, ps, errs[ps])
    say(f"    max-abs error by partition size: {errs}")
    say(f"    raw max-abs by partition size: {raws}")
    return dev, ref


# ------------------------------------------------------------------ the five workloads
def test_tiny_fp32_config():
    run_and_check(W.tiny_case(), partitions=(0, -1, 4, 8, 12))


def test_opt13b_layer_fp16():
    run_and_check(W.opt13b_case(), partitions=(0, -1, 512, 128))


def test_llama7b_shape_reduced():
    case = W.make_decode_case("llama7b_reduced", "llama7b", num_seqs=5, num_heads=32,
                              num_kv_heads=32, head_dim=128, block_size=16,
                              context_lens=[4096, 4096, 3001, 17, 1], kv_dtype="f16",
                              q_dtype="f16", spare_blocks=64)
    run_and_check(case, partitions=(0, -1, 512, 1024))


@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_falcon7b_mqa_fp8(bs):
    ctx = W.falcon7b_lengths(256)
    case = W.make_decode_case(f"falcon7b_fp8_bs{bs}", "falcon7b", num_seqs=256, num_heads=71,
                              num_kv_heads=1, head_dim=64, block_size=bs, context_lens=ctx,
                              kv_dtype="fp8_e4m3", q_dtype="f16",
                              num_blocks=W.falcon7b_num_blocks(ctx, bs))
    run_and_check(case, partitions=(512, 0, -1))


@pytest.mark.parametrize("H", [24, 48])
def test_mqa_fp8_two_workgroups_per_cu(H):
    """64-dimension groups of up to 48 heads run two workgroups per CU: twice the
    workers of the one-workgroup launch, so twice the cut contexts and partial
    records; the Falcon-7B batch (256 sequences of 1..2048 tokens) with 24 heads (two
    16-head tiles, split by quarters) and 48 heads (three whole tiles)."""
    ctx = W.falcon7b_lengths(256)
    case = W.make_decode_case(f"mqa{H}_fp8", "falcon7b", num_seqs=256, num_heads=H,
                              num_kv_heads=1, head_dim=64, block_size=16, context_lens=ctx,
                              kv_dtype="fp8_e4m3", q_dtype="f16",
                              num_blocks=W.falcon7b_num_blocks(ctx, 16), salt=H)
    run_and_check(case, partitions=(-1, 512))


def _llama70b(spec, num_blocks):
    order = W.free_order("llama70b", num_blocks)
    lib_alloc = pa.BlockAllocator(num_blocks, 16, order)
    model = oracle.Allocator(num_blocks, 16, order.tolist())
    case, pairs = W.shared_prompt_case(lib_alloc, spec, num_blocks=num_blocks)
    case_m, pairs_m = W.shared_prompt_case(model, spec, num_blocks=num_blocks)
    # the library allocator and the oracle's model make the same decisions
    assert np.array_equal(case.block_tables, case_m.block_tables)
    assert np.array_equal(case.slot_mapping, case_m.slot_mapping)
    assert np.array_equal(pairs, pairs_m)
    return case, pairs


@pytest.mark.parametrize("full", [False, True])
def test_llama70b_gqa_shared_prompt_cow(full):
    spec = W.llama70b_spec() if full else W.SharedPromptSpec(
        independent_ctx=W.llama70b_independent_lengths(10)[:10] - 1, groups=2, samples=4,
        prompt_len=520)
    case, pairs = _llama70b(spec, 12288 if full else 4096)
    assert len(pairs) == spec.groups * (spec.samples - 1)          # one copy per extra sample
    say(f"[case] llama70b full={full} S={case.num_seqs} cow_pairs={len(pairs)} "
        f"max_ctx={case.max_context_len}")
    # oracle: copy-on-write, write, attention
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    oracle.copy_blocks([kp, vp], [tuple(p) for p in pairs])
    oracle.kv_write(kp, vp, "bf16", case.k_new, case.v_new, "bf16", case.slot_mapping, 16)
    ref = oracle.paged_attention(case.q, "bf16", kp, vp, "bf16", case.block_tables,
                                 case.context_lens, 16, case.scale)
    dev = DeviceCase(case)
    pa.copy_blocks([dev.k_pool], [dev.v_pool], pairs)
    dev.write()
    torch.cuda.synchronize()
    assert_pools_equal(dev, kp, vp)
    for ps in (0, 512, -1):
        out = dev.attend(ps, out=torch.full_like(dev.q, float("nan")))
        torch.cuda.synchronize()
        got = out_to_f64(out)
        err = max_err(got, ref, "bf16")
        say(f"    partition {ps}: max-abs error {err:.3g} (raw {raw_err(got, ref):.3g})")
        assert err <= TOL["bf16"]


def _graph_step_case(kind):
    if kind == "gqa_cow_bf16":
        spec = W.SharedPromptSpec(independent_ctx=W.llama70b_independent_lengths(6)[:6] - 1,
                                  groups=2, samples=3, prompt_len=300)
        return _llama70b(spec, 4096)
    ctx = [0, 1, 17, 300, 700, 64, 129]
    case = W.make_decode_case("graph_mqa_fp8", "tiny", num_seqs=len(ctx), num_heads=71,
                              num_kv_heads=1, head_dim=64, block_size=16, context_lens=ctx,
                              kv_dtype="fp8_e4m3", q_dtype="f16", spare_blocks=8)
    return case, np.zeros((0, 2), dtype=np.int32)


@pytest.mark.parametrize("ps", [0, 512, pa.PARTITION_BALANCED])
@pytest.mark.parametrize("kind", ["gqa_cow_bf16", "mqa_fp8"])
def test_whole_step_graph_replays(kind, ps):
    """One decode step (copy-on-write block copies, cache write, attention)
    captured as one HIP graph and replayed several times; between replays the
    pools are put back to their pre-step bytes eagerly.  Every replay's pools
    match the oracle bit for bit and its output matches the oracle's attention
    and the eager step's output exactly."""
    case, pairs = _graph_step_case(kind)
    say(f"[case] whole-step graph {kind} partition={ps} S={case.num_seqs} pairs={len(pairs)}")
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    if len(pairs):
        oracle.copy_blocks([kp, vp], [tuple(p) for p in pairs])
    oracle.kv_write(kp, vp, case.kv_dtype, case.k_new, case.v_new, case.q_dtype,
                    case.slot_mapping, case.block_size, case.k_scale, case.v_scale)
    ref = oracle.paged_attention(case.q, case.q_dtype, kp, vp, case.kv_dtype, case.block_tables,
                                 case.context_lens, case.block_size, case.scale, case.k_scale,
                                 case.v_scale)
    dev = DeviceCase(case)
    k0, v0 = dev.k_pool.clone(), dev.v_pool.clone()
    need = pa.paged_attention_workspace_size(case.num_seqs, case.num_heads, case.num_kv_heads,
                                             case.head_dim, case.max_context_len, ps)
    ws = pa.new_workspace(need, "cuda")
    out = torch.full_like(dev.q, float("nan"))
    dpairs = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)).cuda()

    def step():
        if len(pairs):
            pa.copy_blocks([dev.k_pool], [dev.v_pool], dpairs)
        dev.write()
        pa.paged_attention_decode(out, dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.ctx,
                                  max_context_len=case.max_context_len, scale=case.scale,
                                  k_scale=case.k_scale, v_scale=case.v_scale,
                                  partition_size=ps, workspace=ws)

    step()
    torch.cuda.synchronize()
    assert_pools_equal(dev, kp, vp)
    eager = out_to_f64(out)
    assert max_err(eager, ref, case.q_dtype) <= TOL[case.kv_dtype]
    dev.k_pool.copy_(k0)
    dev.v_pool.copy_(v0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        dev.k_pool.copy_(k0)
        dev.v_pool.copy_(v0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_pools_equal(dev, kp, vp)
        got = out_to_f64(out)
        err = max_err(got, ref, case.q_dtype)
        say(f"    replay {rep}: max-abs error {err:.3g}")
        assert err <= TOL[case.kv_dtype]
        assert np.array_equal(got, eager), "replay differs from the eager step"
    del g


@pytest.mark.parametrize("kv,q,H,Hkv", [("f16", "f16", 8, 8), ("bf16", "bf16", 64, 8),
                                        ("fp8_e4m3", "bf16", 32, 4)])
def test_pools_beyond_4gib(kv, q, H, Hkv):
    """Pools of about 4.5 GiB each, the case's blocks placed at ids whose byte
    offsets straddle 2 GiB and 4 GiB and at the pool's last block: cache write,
    block copy and attention address them with 64-bit offsets.  Outputs do not
    depend on placement, so the oracle runs on the compact case."""
    ctx = [1, 33, 700, 1500, 16, 0, 2049]
    case = W.make_decode_case(f"big_{kv}_{H}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=128, block_size=16, context_lens=ctx,
                              kv_dtype=kv, q_dtype=q, spare_blocks=2, salt=H)
    kp, vp, ref = oracle_step(case)
    nb = case.k_pool.shape[0]
    block_bytes = Hkv * 16 * 128 * (1 if kv == "fp8_e4m3" else 2)
    NB = (9 << 29) // block_bytes + 2                      # 4.5 GiB and two blocks
    b2, b4 = (1 << 31) // block_bytes, (1 << 32) // block_bytes
    forced = [b2 - 1, b2, b4 - 1, b4, NB - 2, NB - 1]
    rng = np.random.default_rng(nb)
    rest = rng.choice(np.setdiff1d(np.arange(NB - 2), forced), size=nb - len(forced) + 1,
                      replace=False)
    remap = np.concatenate([forced, rest]).astype(np.int64)
    spare = int(remap[-1])                                  # a block no table uses
    remap = remap[:nb]
    rng.shuffle(remap)
    say(f"[case] pools beyond 4 GiB kv={kv} H={H} Hkv={Hkv} NB={NB} "
        f"({NB * block_bytes / 2**30:.2f} GiB per pool)")
    small = DeviceCase(case)
    tdt = small.k_pool.dtype
    idx = torch.from_numpy(remap).cuda()
    big_k = torch.empty((NB, Hkv, 16, 128), dtype=tdt, device="cuda")
    big_v = torch.empty_like(big_k)
    big_k[idx] = small.k_pool
    big_v[idx] = small.v_pool
    tables = np.where(case.block_tables >= 0, remap[np.maximum(case.block_tables, 0)], -1)
    slots = np.where(case.slot_mapping >= 0,
                     remap[np.maximum(case.slot_mapping, 0) // 16] * 16 + case.slot_mapping % 16,
                     -1)
    tables_d = torch.from_numpy(tables.astype(np.int32)).cuda()
    pa.kv_cache_write(small.k_new, small.v_new, big_k, big_v,
                      torch.from_numpy(slots.astype(np.int64)).cuda(),
                      k_scale=case.k_scale, v_scale=case.v_scale)
    torch.cuda.synchronize()
    gk, gv = from_dev(big_k[idx], kv), from_dev(big_v[idx], kv)
    assert np.array_equal(W.raw_view(gk, kv), W.raw_view(kp, kv)), "K pool differs after write"
    assert np.array_equal(W.raw_view(gv, kv), W.raw_view(vp, kv)), "V pool differs after write"
    for ps in (0, pa.PARTITION_BALANCED, 512):
        out = torch.full_like(small.q, float("nan"))
        pa.paged_attention_decode(out, small.q, big_k, big_v, tables_d, small.ctx,
                                  max_context_len=case.max_context_len, scale=case.scale,
                                  k_scale=case.k_scale, v_scale=case.v_scale, partition_size=ps)
        torch.cuda.synchronize()
        err = max_err(out_to_f64(out), ref, q)
        say(f"    partition {ps}: max-abs error {err:.3g}")
        assert err <= TOL[kv]
    # copy the block at the 4 GiB boundary and the last block to the spare one and back
    for src in (b4, NB - 1):
        before = from_dev(big_k[src], kv).copy()
        pa.copy_blocks([big_k], [big_v], [(src, spare)])
        torch.cuda.synchronize()
        assert np.array_equal(W.raw_view(from_dev(big_k[spare], kv), kv), W.raw_view(before, kv))
        assert np.array_equal(W.raw_view(from_dev(big_v[spare], kv), kv),
                              W.raw_view(from_dev(big_v[src], kv), kv))
    del big_k, big_v
    torch.cuda.empty_cache()


def test_serving_loop_many_steps():
    """24 decode steps as a server runs them: the library allocator and the
    oracle's model in lockstep (same tables, slots and copy pairs), prompts
    written through the cache write, parallel samples forked from partly
    filled blocks (copy-on-write at their next write), a sequence freed and a
    new one admitted into reused blocks.  Every step: block copies, cache write
    and attention on the GPU; the pools match the oracle's bit for bit and the
    output matches its attention.  Modes cycle through single pass, balanced
    and partitions."""
    NB, Hkv, H, D, bs = 96, 2, 8, 64, 8
    rng = np.random.default_rng(2024)
    order = rng.permutation(NB).astype(np.int32)
    lib_alloc = pa.BlockAllocator(NB, bs, order)
    model = oracle.Allocator(NB, bs, order.tolist())
    kp = W.empty_pool(NB, Hkv, bs, D, "bf16")
    vp = W.empty_pool(NB, Hkv, bs, D, "bf16")
    dk, dv = to_dev(kp, "bf16"), to_dev(vp, "bf16")
    scale = 1.0 / math.sqrt(D)

    def vals(*shape):
        return W.to_storage(rng.standard_normal(shape).astype(np.float32), "bf16")

    def write(slots, kn, vn):
        oracle.kv_write(kp, vp, "bf16", kn, vn, "bf16", slots, bs)
        pa.kv_cache_write(to_dev(kn, "bf16"), to_dev(vn, "bf16"), dk, dv,
                          torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda())

    def admit(sid, prompt):
        lib_alloc.add_seq(sid, prompt)
        model.add_seq(sid, prompt)
        slots = [model.slot(sid, t) for t in range(prompt)]
        assert slots == [lib_alloc.physical_block(sid, t // bs) * bs + t % bs
                         for t in range(prompt)]
        write(slots, vals(prompt, Hkv, D), vals(prompt, Hkv, D))

    def fork(parent, child):
        lib_alloc.fork(parent, child)
        model.fork(parent, child)

    def free(sid):
        lib_alloc.free_seq(sid)
        model.free_seq(sid)

    live = [0, 1, 2]
    for sid, prompt in zip(live, (5, 8, 17)):
        admit(sid, prompt)
    events = {2: lambda: (fork(0, 10), fork(0, 11), live.extend([10, 11])),
              10: lambda: (free(1), live.remove(1), admit(3, 12), live.append(3)),
              16: lambda: (fork(3, 12), live.append(12)),
              20: lambda: (free(10), live.remove(10))}
    copies = 0
    for step in range(24):
        if step in events:
            events[step]()
        slots, pairs = lib_alloc.append_slots(live)
        m_slots, m_pairs = model.append_slots(live)
        assert slots.tolist() == list(m_slots)
        assert [tuple(p) for p in pairs.tolist()] == [tuple(p) for p in m_pairs]
        copies += len(pairs)
        if len(pairs):
            oracle.copy_blocks([kp, vp], [tuple(p) for p in pairs.tolist()])
            pa.copy_blocks([dk], [dv], pairs)
        write(slots.tolist(), vals(len(live), Hkv, D), vals(len(live), Hkv, D))
        max_blocks = 8
        tables, lens = lib_alloc.export(live, max_blocks)
        m_tables, m_lens = model.export(live, max_blocks)
        assert np.array_equal(tables, m_tables) and np.array_equal(lens, m_lens)
        q = vals(len(live), H, D)
        ref = oracle.paged_attention(q, "bf16", kp, vp, "bf16", tables, lens, bs, scale)
        ps = (0, pa.PARTITION_BALANCED, 16)[step % 3]
        out = torch.full((len(live), H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        pa.paged_attention_decode(out, to_dev(q, "bf16"), dk, dv,
                                  torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                                  max_context_len=int(lens.max()), scale=scale,
                                  partition_size=ps)
        torch.cuda.synchronize()
        assert np.array_equal(W.raw_view(from_dev(dk, "bf16"), "bf16"), W.raw_view(kp, "bf16"))
        assert np.array_equal(W.raw_view(from_dev(dv, "bf16"), "bf16"), W.raw_view(vp, "bf16"))
        err = max_err(out_to_f64(out), ref, "bf16")
        say(f"    step {step}: live {live} lens {lens.tolist()} pairs {len(pairs)} "
            f"partition {ps} max-abs error {err:.3g}")
        assert err <= TOL["bf16"]
    assert copies >= 3          # the forks from partly filled blocks were copied on write


def test_side_stream_without_workspace():
    """A call on a side stream with no workspace: the binding allocates the
    partial records in that stream's order, so memory the current stream takes
    (and overwrites) right after the call cannot be the records the kernels are
    still using.  Balanced and partitioned modes (both write records), checked
    against the oracle after the current stream has filled fresh allocations."""
    case = W.make_decode_case("side_stream", "tiny", num_seqs=48, num_heads=16, num_kv_heads=2,
                              head_dim=128, block_size=16,
                              context_lens=np.random.default_rng(7).integers(300, 3000, 48).tolist(),
                              kv_dtype="bf16", q_dtype="bf16", spare_blocks=5, salt=7)
    kp, vp, ref = oracle_step(case)
    dev = DeviceCase(case)
    dev.write()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say("[case] side stream, no workspace")
    for ps in (pa.PARTITION_BALANCED, 256):
        out = torch.full_like(dev.q, float("nan"))
        side.wait_stream(torch.cuda.current_stream())
        pa.paged_attention_decode(out, dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.ctx,
                                  max_context_len=case.max_context_len, scale=case.scale,
                                  partition_size=ps, stream=side)
        # the current stream allocates and writes straight away, while the side
        # stream's kernels may still run
        junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(64)]
        side.synchronize()
        torch.cuda.synchronize()
        del junk
        err = max_err(out_to_f64(out), ref, case.q_dtype)
        say(f"    partition {ps}: max-abs error {err:.3g}")
        assert err <= TOL[case.kv_dtype], (ps, err)


def test_two_threads_two_streams():
    """Two host threads, each with its own stream and workspace, run cache
    writes and attention on different cases at the same time (the library
    keeps no device state between calls; its host caches are locked).  Both
    match the oracle in every mode."""
    import threading
    cases = [W.make_decode_case("threads_gqa", "tiny", num_seqs=40, num_heads=16, num_kv_heads=2,
                                head_dim=128, block_size=16,
                                context_lens=np.random.default_rng(1).integers(1, 900, 40).tolist(),
                                kv_dtype="bf16", q_dtype="bf16", spare_blocks=5, salt=1),
             W.make_decode_case("threads_mha", "tiny", num_seqs=24, num_heads=8, num_kv_heads=8,
                                head_dim=64, block_size=32,
                                context_lens=np.random.default_rng(2).integers(0, 1500, 24).tolist(),
                                kv_dtype="fp8_e4m3", q_dtype="f16", spare_blocks=5, salt=2)]
    refs = [oracle_step(c) for c in cases]
    devs = [DeviceCase(c) for c in cases]
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(i):
        try:
            c, d = cases[i], devs[i]
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                pa.kv_cache_write(d.k_new, d.v_new, d.k_pool, d.v_pool, d.slots,
                                  k_scale=c.k_scale, v_scale=c.v_scale, stream=st)
                for rep in range(4):
                    for ps in (0, pa.PARTITION_BALANCED, 256):
                        need = pa.paged_attention_workspace_size(
                            c.num_seqs, c.num_heads, c.num_kv_heads, c.head_dim,
                            c.max_context_len, ps)
                        ws = pa.new_workspace(need, "cuda")
                        out = torch.full_like(d.q, float("nan"))
                        pa.paged_attention_decode(out, d.q, d.k_pool, d.v_pool, d.tables, d.ctx,
                                                  max_context_len=c.max_context_len,
                                                  scale=c.scale, k_scale=c.k_scale,
                                                  v_scale=c.v_scale, partition_size=ps,
                                                  workspace=ws, stream=st)
                        results[(i, rep, ps)] = out
            st.synchronize()
        except Exception as e:              # reported by the main thread
            errors.append(repr(e))

    say("[case] two threads, two streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (c, d) in enumerate(zip(cases, devs)):
        kp, vp, ref = refs[i]
        assert_pools_equal(d, kp, vp)
        for (j, rep, ps), out in results.items():
            if j == i:
                err = max_err(out_to_f64(out), ref, c.q_dtype)
                assert err <= TOL[c.kv_dtype], (c.name, rep, ps, err)
    say(f"    {len(results)} launches checked")


def test_llama7b_full_size_sampled():
    """64 sequences at context 4096, 17,408-block pool (4 GiB per layer): GPU writes
    and attends over the whole batch; the oracle recomputes sampled sequences from
    the pre-write bytes of their blocks."""
    ctx = np.full(64, 4096, dtype=np.int32)
    say("[case] llama7b full size: generating 2 x 2.1 GiB pools on device")
    d = W.device_pool_case("llama7b_full", "llama7b", num_seqs=64, num_heads=32, num_kv_heads=32,
                           head_dim=128, block_size=16, context_lens=ctx, kv_dtype="f16",
                           num_blocks=17408)
    sampled = [0, 17, 42, 63]
    nblk = 256
    pre_k = {s: d["k_pool"][torch.from_numpy(d["tables"][s, :nblk]).long().cuda()].cpu().numpy()
             for s in sampled}
    pre_v = {s: d["v_pool"][torch.from_numpy(d["tables"][s, :nblk]).long().cuda()].cpu().numpy()
             for s in sampled}
    slots = torch.from_numpy(d["slots"]).cuda()
    pa.kv_cache_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], slots)
    tables = torch.from_numpy(d["tables"]).cuda()
    ctx_t = torch.from_numpy(ctx).cuda()
    outs = {}
    for ps in (0, 512, -1):
        out = torch.full_like(d["q"], float("nan"))
        pa.paged_attention_decode(out, d["q"], d["k_pool"], d["v_pool"], tables, ctx_t,
                                  max_context_len=4096, scale=d["scale"], partition_size=ps)
        torch.cuda.synchronize()
        outs[ps] = out_to_f64(out)
        assert np.isfinite(outs[ps]).all()
    qh = d["q"].cpu().numpy()
    kn, vn = d["k_new"].cpu().numpy(), d["v_new"].cpu().numpy()
    for s in sampled:
        kp, vp = pre_k[s].copy(), pre_v[s].copy()
        local_table = np.arange(nblk, dtype=np.int32)[None, :]
        slot = np.array([(nblk - 1) * 16 + 15])
        oracle.kv_write(kp, vp, "f16", kn[s:s + 1], vn[s:s + 1], "f16", slot, 16)
        ref = oracle.paged_attention(qh[s:s + 1], "f16", kp, vp, "f16", local_table,
                                     [4096], 16, d["scale"])[0]
        # the GPU-written slot holds the same bits as the oracle's
        blk = int(d["tables"][s, nblk - 1])
        got_k = d["k_pool"][blk, :, 15, :].cpu().numpy()
        assert np.array_equal(got_k.view(np.uint16), kp[nblk - 1, :, 15, :].view(np.uint16))
        for ps, o in outs.items():
            err = max_err(o[s], ref, "f16")
            say(f"    seq {s} partition {ps}: max-abs error {err:.3g}")
            assert err <= TOL["f16"]
    del d


def test_llama7b_full_step_every_sequence_layer():
    """The whole Llama-2-7B decode step in its timed launch configuration: 32 layers,
    each with its own 17,408-block pools (4.25 GiB of K+V per layer, one block table
    for all layers), 64 sequences at context 4096, per layer the cache write and then
    single-pass attention with a caller workspace.  Every one of the 2,048
    sequence-layers is recomputed by the oracle from its blocks as the step left them
    (the oracle rewrites the new token's slot, whose bytes must already be the GPU's)."""
    import concurrent.futures as cf
    S, H, Hkv, D, bs, NB, L = 64, 32, 32, 128, 16, 17408, 32
    nblk = 4096 // bs
    ctx = np.full(S, 4096, dtype=np.int32)
    say(f"[case] llama7b full step: {L} layers of 4.25 GiB pools on device")
    layers = [W.device_pool_case(f"llama7b_l{l}", "llama7b", num_seqs=S, num_heads=H,
                                 num_kv_heads=Hkv, head_dim=D, block_size=bs, context_lens=ctx,
                                 kv_dtype="f16", num_blocks=NB, layer=l, place_layer=0)
              for l in range(L)]
    tab = layers[0]["tables"]
    tables = torch.from_numpy(tab).cuda()
    ctx_t = torch.from_numpy(ctx).cuda()
    slots = torch.from_numpy(layers[0]["slots"]).cuda()
    ws = pa.new_workspace(pa.paged_attention_workspace_size(S, H, Hkv, D, 4096, 0), "cuda")
    for d in layers:
        d["out"] = torch.full_like(d["q"], float("nan"))
        pa.kv_cache_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], slots)
        pa.paged_attention_decode(d["out"], d["q"], d["k_pool"], d["v_pool"], tables, ctx_t,
                                  max_context_len=4096, scale=d["scale"], partition_size=0,
                                  workspace=ws)
    torch.cuda.synchronize()
    scale = layers[0]["scale"]
    host = [dict(q=d["q"].cpu().numpy(), kn=d["k_new"].cpu().numpy(), vn=d["v_new"].cpu().numpy(),
                 out=out_to_f64(d["out"])) for d in layers]
    local = np.arange(nblk, dtype=np.int32)[None, :]
    slot = np.array([(nblk - 1) * bs + (4095 % bs)])

    def check(x):
        l, s, kp, vp = x
        h = host[l]
        got_k, got_v = kp[nblk - 1, :, 4095 % bs, :].copy(), vp[nblk - 1, :, 4095 % bs, :].copy()
        oracle.kv_write(kp, vp, "f16", h["kn"][s:s + 1], h["vn"][s:s + 1], "f16", slot, bs)
        same = (np.array_equal(got_k.view(np.uint16), kp[nblk - 1, :, 4095 % bs, :].view(np.uint16)) and
                np.array_equal(got_v.view(np.uint16), vp[nblk - 1, :, 4095 % bs, :].view(np.uint16)))
        ref = oracle.paged_attention(h["q"][s:s + 1], "f16", kp, vp, "f16", local, [4096], bs, scale)[0]
        return l, s, same, bool(np.isfinite(h["out"][s]).all()), max_err(h["out"][s], ref, "f16")

    work = [(l, s) for l in range(L) for s in range(S)]
    results = []
    with cf.ThreadPoolExecutor(16) as ex:
        for i in range(0, len(work), 16):
            xs = []
            for l, s in work[i:i + 16]:
                idx = torch.from_numpy(tab[s, :nblk].astype(np.int64)).cuda()
                xs.append((l, s, layers[l]["k_pool"][idx].cpu().numpy(),
                           layers[l]["v_pool"][idx].cpu().numpy()))
            results += list(ex.map(check, xs))
    worst = max(results, key=lambda r: r[4])
    say(f"    {len(results)} sequence-layers: worst max-abs error {worst[4]:.3g} "
        f"(layer {worst[0]}, sequence {worst[1]})")
    assert all(r[2] for r in results), "a written slot differs from the oracle's encoding"
    assert all(r[3] for r in results)
    assert worst[4] <= TOL["f16"]
    del layers, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16, 64 << 20])
def test_stream_read_reads_every_word(nbytes):
    """The read-rate probe visits every 16-byte piece once: the XOR of its sink words
    equals the XOR of the buffer's words."""
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda",
                        generator=g)
    sink = torch.zeros(pa.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    pa.stream_read(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_stream_read_refuses_ranges_past_the_allocation():
    """A range longer than any allocation, and memory HIP does not know, are refused on
    the host (nothing is enqueued).  (torch's caching allocator carves tensors out of
    larger segments, so a range just past a tensor's end may still lie inside one.)"""
    import ctypes
    buf = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(pa.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    read = pa.lib.pa_stream_read
    assert read(ctypes.c_void_p(buf.data_ptr()), 64 << 20, ctypes.c_void_p(sink.data_ptr()), s) == 0
    assert read(ctypes.c_void_p(buf.data_ptr()), 1 << 40, ctypes.c_void_p(sink.data_ptr()), s) == -1
    host = np.zeros(1 << 16, dtype=np.uint8)
    assert read(ctypes.c_void_p(host.ctypes.data), 16, ctypes.c_void_p(sink.data_ptr()), s) == -1
    assert read(ctypes.c_void_p(buf.data_ptr()), 16, ctypes.c_void_p(host.ctypes.data), s) == -1
    torch.cuda.synchronize()


# ------------------------------------------------------------------ edge cases
EDGE = [
    # kv, q, D, bs, H, Hkv, ctx
    ("f32", "f32", 64, 1, 2, 1, [0, 1, 2, 37]),
    ("f32", "f32", 128, 2, 4, 4, [3, 64, 65]),
    ("f16", "f16", 64, 4, 6, 3, [1, 4, 5, 300]),
    ("f16", "f16", 128, 32, 8, 2, [31, 32, 33, 513]),
    ("bf16", "bf16", 64, 64, 4, 1, [63, 64, 65, 700]),
    ("bf16", "bf16", 128, 128, 2, 2, [1, 127, 129, 1025]),
    ("f16", "f16", 128, 256, 4, 2, [255, 256, 600]),
    ("fp8_e4m3", "f16", 128, 16, 4, 2, [1, 16, 17, 333]),
    ("fp8_e4m3", "bf16", 64, 8, 8, 8, [2, 9, 1000]),
    ("fp8_e4m3", "f32", 64, 32, 3, 1, [5, 40, 97]),
    # items longer than a wavefront's staged block-table slice (256 entries)
    ("f16", "f16", 128, 1, 4, 4, [1, 700, 2100]),
    ("f32", "f32", 64, 4, 2, 2, [4100, 3]),
    ("bf16", "bf16", 128, 2, 8, 2, [600, 1500]),
    ("fp8_e4m3", "f16", 64, 1, 71, 1, [300, 1100]),
]


@pytest.mark.parametrize("kv,q,D,bs,H,Hkv,ctx", EDGE)
def test_edge_shapes(kv, q, D, bs, H, Hkv, ctx):
    case = W.make_decode_case(f"edge_{kv}_{D}_{bs}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=D, block_size=bs, context_lens=ctx,
                              kv_dtype=kv, q_dtype=q, spare_blocks=5, salt=bs + D,
                              max_blocks=int(W.blocks_needed(ctx, bs).max()) + 3)
    run_and_check(case, partitions=(0, -1, 3 * bs, 100))


def test_empty_batch_and_empty_contexts():
    case = W.make_decode_case("empty", "tiny", num_seqs=3, num_heads=2, num_kv_heads=2,
                              head_dim=64, block_size=16, context_lens=[0, 0, 5], kv_dtype="f16",
                              q_dtype="f16", spare_blocks=2, append=False)
    dev = DeviceCase(case)
    say("[case] empty contexts")
    for ps in (0, 16, -1):
        out = dev.attend(ps, out=torch.full_like(dev.q, float("nan")))
        torch.cuda.synchronize()
        o = out_to_f64(out)
        assert np.array_equal(o[:2], np.zeros_like(o[:2]))
        ref = oracle.paged_attention(case.q, "f16", case.k_pool, case.v_pool, "f16",
                                     case.block_tables, case.context_lens, 16, case.scale)
        assert max_err(o, ref, "f16") <= TOL["f16"]


def test_placement_permutation_is_bit_identical():
    """Summation order depends only on logical order: relocating blocks changes nothing."""
    case = W.make_decode_case("perm", "tiny", num_seqs=4, num_heads=8, num_kv_heads=8,
                              head_dim=128, block_size=16, context_lens=[100, 1000, 7, 64],
                              kv_dtype="f16", q_dtype="f16", spare_blocks=40, append=False)
    say("[case] placement permutation")
    a = DeviceCase(case).attend(0).clone()
    a_split = DeviceCase(case).attend(256).clone()
    a_bal = DeviceCase(case).attend(-1).clone()
    perm = np.random.default_rng(1).permutation(case.num_blocks)
    k2 = np.empty_like(case.k_pool); v2 = np.empty_like(case.v_pool)
    k2[perm] = case.k_pool; v2[perm] = case.v_pool
    case.k_pool, case.v_pool = k2, v2
    case.block_tables = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)],
                                 -1).astype(np.int32)
    b = DeviceCase(case).attend(0)
    b_split = DeviceCase(case).attend(256)
    b_bal = DeviceCase(case).attend(-1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a_split.view(torch.int16), b_split.view(torch.int16))
    assert torch.equal(a_bal.view(torch.int16), b_bal.view(torch.int16))


def test_invalid_table_entries_are_never_read():
    case = W.make_decode_case("badtable", "tiny", num_seqs=2, num_heads=2, num_kv_heads=2,
                              head_dim=64, block_size=4, context_lens=[12, 9], kv_dtype="f32",
                              q_dtype="f32", spare_blocks=3, append=False)
    good = case.block_tables.copy()
    case.block_tables[0, 1] = -7
    case.block_tables[1, 2] = case.num_blocks + 1000
    say("[case] invalid table entries")
    out = out_to_f64(DeviceCase(case).attend(0))
    Q = case.q.astype(np.float64)
    for s, skip in ((0, 1), (1, 2)):
        n = int(case.context_lens[s])
        keep = [t for t in range(n) if t // 4 != skip]
        K = oracle.gather_sequence(case.k_pool, "f32", good[s], n, 4)[keep]
        V = oracle.gather_sequence(case.v_pool, "f32", good[s], n, 4)[keep]
        ref = oracle.contiguous_attention(Q[s], K, V, case.scale)
        assert max_err(out[s], ref, "f32") <= TOL["f32"]


def test_context_clamped_to_max_context_len():
    case = W.make_decode_case("clamp", "tiny", num_seqs=2, num_heads=2, num_kv_heads=2,
                              head_dim=64, block_size=8, context_lens=[50, 20], kv_dtype="f16",
                              q_dtype="f16", spare_blocks=3, append=False)
    dev = DeviceCase(case)
    say("[case] clamp to max_context_len")
    out = torch.empty_like(dev.q)
    pa.paged_attention_decode(out, dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.ctx,
                              max_context_len=30, scale=case.scale)
    torch.cuda.synchronize()
    ref = oracle.paged_attention(case.q, "f16", case.k_pool, case.v_pool, "f16",
                                 case.block_tables, [30, 20], 8, case.scale)
    assert max_err(out_to_f64(out), ref, "f16") <= TOL["f16"]


# ------------------------------------------------------------------ cache write, block copy
@pytest.mark.parametrize("src", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("scale", [1.0, 0.125, 3.7])
def test_fp8_write_bit_exact_exhaustive(src, scale):
    """Every fp16 (or bf16) bit pattern, and random fp32 values, quantised by the
    cache write must give the oracle's e4m3 codes bit for bit."""
    Hkv, D, bs = 1, 64, 16
    if src == "f32":
        rng = np.random.default_rng(3)
        vals = (np.exp2(rng.uniform(-20, 12, 65536)) * rng.choice([-1, 1], 65536)).astype(np.float32)
        vals[:6] = [np.inf, -np.inf, np.nan, 0.0, -0.0, 448.0]
        new = vals
    else:
        new = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        if src == "f16":
            new = new.view(np.float16)
    T = 65536 // (Hkv * D)
    new = new.reshape(T, Hkv, D)
    NB = T // bs + 4
    slots = np.random.default_rng(4).permutation(NB * bs)[:T].astype(np.int64)
    kp = W.empty_pool(NB, Hkv, bs, D, "fp8_e4m3")
    vp = W.empty_pool(NB, Hkv, bs, D, "fp8_e4m3")
    say(f"[case] fp8 write exhaustive src={src} scale={scale}")
    gk, gv = to_dev(kp, "fp8_e4m3"), to_dev(vp, "fp8_e4m3")
    nd = to_dev(new, src)
    nd_v = to_dev(new[::-1].copy(), src)
    pa.kv_cache_write(nd, nd_v, gk, gv, torch.from_numpy(slots).cuda(), k_scale=scale,
                      v_scale=scale * 2)
    torch.cuda.synchronize()
    oracle.kv_write(kp, vp, "fp8_e4m3", new, new[::-1].copy(), src, slots, bs, scale, scale * 2)
    assert np.array_equal(from_dev(gk, "fp8_e4m3"), kp)
    assert np.array_equal(from_dev(gv, "fp8_e4m3"), vp)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_write_bit_exact_same_dtype_with_skips(dt):
    case = W.make_decode_case(f"write_{dt}", "tiny", num_seqs=40, num_heads=4, num_kv_heads=4,
                              head_dim=128, block_size=16, context_lens=list(range(1, 41)),
                              kv_dtype=dt, q_dtype="f16" if dt == "fp8_e4m3" else dt,
                              spare_blocks=3)
    case.slot_mapping[::5] = -1
    case.slot_mapping[3] = case.num_blocks * 16 + 99        # out of range: skipped
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    oracle.kv_write(kp, vp, dt, case.k_new, case.v_new, dt, case.slot_mapping, 16)
    dev = DeviceCase(case)
    say(f"[case] write {dt}")
    dev.write()
    torch.cuda.synchronize()
    assert_pools_equal(dev, kp, vp)


@pytest.mark.parametrize("dt", ["f16", "fp8_e4m3", "f32"])
def test_copy_blocks_bit_exact_many_layers_and_pairs(dt):
    L, NB, Hkv, bs, D = 37, 200, 2, 16, 64
    rng = np.random.default_rng(7)
    storage = W.STORAGE[dt]
    pools_np = []
    for _ in range(2 * L):
        raw = rng.integers(0, 255, size=(NB, Hkv, bs, D * W.ELEM_BYTES[dt]), dtype=np.uint8)
        pools_np.append(raw.view(storage).reshape(NB, Hkv, bs, D))
    perm = rng.permutation(NB)
    pairs = np.stack([perm[:70], perm[70:140]], axis=1).astype(np.int32)   # 70 pairs
    say(f"[case] copy_blocks {dt} layers={L} pairs={len(pairs)}")
    dev = [to_dev(p, dt) for p in pools_np]
    pa.copy_blocks(dev[:L], dev[L:], pairs)
    torch.cuda.synchronize()
    oracle.copy_blocks(pools_np, [tuple(p) for p in pairs])
    for g, r in zip(dev, pools_np):
        assert np.array_equal(W.raw_view(from_dev(g, dt), dt), W.raw_view(r, dt))


def test_copy_blocks_device_pairs_skip_padding():
    """Pairs read from device memory: rows with an id outside the pool (-1
    padding, >= num_blocks) or with src == dst are skipped; the rest are
    copied bit for bit."""
    L, NB, Hkv, bs, D, dt = 3, 64, 2, 16, 64, "bf16"
    rng = np.random.default_rng(11)
    pools_np = [rng.integers(0, 65535, size=(NB, Hkv, bs, D), dtype=np.uint16) for _ in range(2 * L)]
    pairs = np.array([[3, 9], [-1, -1], [5, 70], [4, 4], [12, 1], [-1, 20], [63, 0]], np.int32)
    dev = [to_dev(p, dt) for p in pools_np]
    say(f"[case] copy_blocks device pairs with padding rows={len(pairs)}")
    pa.copy_blocks(dev[:L], dev[L:], torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    oracle.copy_blocks(pools_np, [(3, 9), (12, 1), (63, 0)])
    for g, r in zip(dev, pools_np):
        assert np.array_equal(from_dev(g, dt), r)


def test_copy_blocks_graph_replays_new_pairs():
    """One captured copy_blocks launch over a fixed-capacity device pair buffer,
    replayed with two different pair sets written into the buffer between
    replays (the copy-on-write pairs of two different steps): each replay is
    bit-exact against the oracle's block copy of that step's pairs."""
    L, NB, Hkv, bs, D, dt, cap = 4, 96, 2, 16, 128, "f16", 16
    rng = np.random.default_rng(12)
    base = [rng.integers(0, 65535, size=(NB, Hkv, bs, D), dtype=np.uint16).view(np.float16)
            for _ in range(2 * L)]
    dev = [to_dev(p, dt) for p in base]
    buf = torch.full((cap, 2), -1, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        pa.copy_blocks(dev[:L], dev[L:], buf)
    perm = rng.permutation(NB)
    steps = [np.stack([perm[:5], perm[5:10]], axis=1), np.stack([perm[20:31], perm[40:51]], axis=1)]
    for i, pairs in enumerate(steps):
        host = np.full((cap, 2), -1, np.int32)
        host[:len(pairs)] = pairs
        buf.copy_(torch.from_numpy(host))
        for d, b in zip(dev, base):
            d.copy_(torch.from_numpy(b))
        torch.cuda.synchronize()
        say(f"[case] copy_blocks graph replay {i} pairs={len(pairs)}")
        g.replay()
        torch.cuda.synchronize()
        ref = [b.copy() for b in base]
        oracle.copy_blocks(ref, [tuple(p) for p in pairs.tolist()])
        for d, r in zip(dev, ref):
            assert np.array_equal(from_dev(d, dt).view(np.uint16), r.view(np.uint16)), i


# ------------------------------------------------------------------ grouped heads (matrix-core path)
MFMA_CASES = [
    # kv, q, D, bs, H, Hkv, ctx
    ("bf16", "bf16", 128, 16, 64, 8, [1, 17, 31, 32, 33, 530, 1000]),
    ("f16", "f16", 128, 16, 32, 2, [5, 64, 700]),
    ("f16", "f16", 64, 8, 12, 1, [3, 100, 257]),
    ("bf16", "bf16", 64, 32, 10, 2, [2, 33, 129]),
    ("f16", "f16", 128, 64, 6, 2, [65, 128, 400]),
    ("bf16", "bf16", 128, 4, 8, 4, [9, 50]),
    ("fp8_e4m3", "f16", 64, 16, 16, 2, [1, 40, 600]),
    ("fp8_e4m3", "bf16", 128, 16, 16, 2, [7, 300]),
    ("fp8_e4m3", "f16", 128, 32, 24, 2, [31, 90]),
    ("f16", "f16", 128, 1, 4, 2, [1, 2, 45]),
    # G > 16: a workgroup per KV head, K/V staged once in LDS; tiles of 16 heads taken
    # whole by one wavefront, or by four that take a quarter of every step each and
    # merge (2 and 5 tiles); 3, 4, 6, 7, 8 tiles and a last tile with one head
    ("fp8_e4m3", "f16", 64, 16, 71, 1, [1, 2, 31, 32, 33, 700, 2048]),
    ("fp8_e4m3", "bf16", 64, 16, 40, 1, [3, 64, 65, 500]),
    ("bf16", "bf16", 128, 16, 90, 1, [1, 300]),
    ("f16", "f16", 64, 8, 34, 2, [2, 130, 777]),
    ("fp8_e4m3", "bf16", 64, 32, 80, 1, [63, 64, 65, 1200]),
    ("fp8_e4m3", "bf16", 64, 8, 71, 1, [5, 100, 513]),
    ("f16", "f16", 128, 16, 64, 2, [17, 300]),
    ("bf16", "bf16", 128, 32, 64, 1, [1, 64, 200]),
    ("bf16", "bf16", 64, 16, 20, 1, [9, 77]),
    ("f16", "f16", 64, 64, 128, 1, [3, 130]),
    ("fp8_e4m3", "f16", 128, 16, 100, 1, [40, 129]),
]


@pytest.mark.parametrize("kv,q,D,bs,H,Hkv,ctx", MFMA_CASES)
def test_grouped_heads(kv, q, D, bs, H, Hkv, ctx):
    case = W.make_decode_case(f"gqa_{kv}_{q}_{D}_{bs}_{H}x{Hkv}", "tiny", num_seqs=len(ctx),
                              num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                              context_lens=ctx, kv_dtype=kv, q_dtype=q, spare_blocks=7,
                              salt=H * 7 + bs, max_blocks=int(W.blocks_needed(ctx, bs).max()) + 2)
    run_and_check(case, partitions=(0, -1, 64, 512))


@pytest.mark.parametrize("H,Hkv,D", [(8, 1, 64), (16, 4, 128), (71, 1, 64), (40, 2, 128), (8, 8, 128)])
def test_fp8_cache_bf16_queries_beyond_fp16_range(H, Hkv, D):
    """bf16 queries whose entries reach ~1e5 .. 1e6 (fp16 stops at 65504) over an
    fp8 cache: the codes are widened to the query's type, so the queries are used
    as they are.  The queries are the seeded ones times 2^18 (exact in bf16) and
    the softmax scale is divided by 2^18, so the weights stay those of ordinary
    inputs and the comparison keeps the fp8 tolerance."""
    ctx = [1, 37, 300, 1025]
    case = W.make_decode_case(f"fp8_bigq_{H}x{Hkv}_{D}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=D, block_size=16, context_lens=ctx,
                              kv_dtype="fp8_e4m3", q_dtype="bf16", spare_blocks=5, salt=H + D)
    f = torch.from_numpy(case.q.copy()).view(torch.bfloat16).float() * float(2 ** 18)
    big = f.to(torch.bfloat16)
    assert torch.equal(big.float(), f)                               # the scaling is exact
    assert float(big.float().abs().max()) > 65504.0
    case = dataclasses.replace(case, q=big.view(torch.int16).numpy().view(np.uint16),
                               scale=case.scale / 2 ** 18)
    run_and_check(case, partitions=(0, -1, 512))


def test_grouped_heads_invalid_table_entries():
    case = W.make_decode_case("gqa_badtable", "tiny", num_seqs=2, num_heads=16, num_kv_heads=2,
                              head_dim=128, block_size=16, context_lens=[100, 70], kv_dtype="bf16",
                              q_dtype="bf16", spare_blocks=3, append=False)
    good = case.block_tables.copy()
    case.block_tables[0, 2] = -1
    case.block_tables[1, 1] = case.num_blocks + 7
    say("[case] grouped heads, invalid table entries")
    out = out_to_f64(DeviceCase(case).attend(0))
    Q = oracle.decode(case.q, "bf16")
    for s, skip in ((0, 2), (1, 1)):
        n = int(case.context_lens[s])
        keep = [t for t in range(n) if t // 16 != skip]
        K = oracle.gather_sequence(case.k_pool, "bf16", good[s], n, 16)[keep]
        V = oracle.gather_sequence(case.v_pool, "bf16", good[s], n, 16)[keep]
        ref = oracle.contiguous_attention(Q[s], K, V, case.scale)
        assert max_err(out[s], ref, "bf16") <= TOL["bf16"]


# ------------------------------------------------------------------ work sharing across launches
WINDOW_CASES = [
    # kv, q, H, Hkv (one case per decode kernel: per-head, grouped-head, large group)
    ("f16", "f16", 4, 4),
    ("bf16", "bf16", 8, 2),
    ("fp8_e4m3", "f16", 32, 1),
]


@pytest.mark.parametrize("kv,q,H,Hkv", WINDOW_CASES)
def test_many_windows_and_workspace_reuse(kv, q, H, Hkv):
    """2500 sequences span three 1024-sequence windows of the schedule; one
    workspace serves several eager launches and graph replays, which all agree
    bit for bit."""
    rng = np.random.default_rng(7)
    ctx = rng.integers(0, 70, size=2500)
    ctx[::97] = 0
    ctx[5] = 400
    case = W.make_decode_case(f"windows_{kv}_{H}_{Hkv}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=64, block_size=16,
                              context_lens=ctx.tolist(), kv_dtype=kv, q_dtype=q, spare_blocks=7,
                              append=False)
    dev = DeviceCase(case)
    say(f"[case] windows kv={kv} q={q} H={H} Hkv={Hkv}")
    ref = oracle.paged_attention(case.q, q, case.k_pool, case.v_pool, kv, case.block_tables,
                                 case.context_lens, 16, case.scale, case.k_scale, case.v_scale)
    for ps in (0, 32, pa.PARTITION_BALANCED):
        need = pa.paged_attention_workspace_size(len(ctx), H, Hkv, 64, case.max_context_len, ps)
        ws = pa.new_workspace(need, "cuda")
        outs = []

        def launch(out):
            pa.paged_attention_decode(out, dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.ctx,
                                      max_context_len=case.max_context_len, scale=case.scale,
                                      k_scale=case.k_scale, v_scale=case.v_scale,
                                      partition_size=ps, workspace=ws)

        for _ in range(3):
            out = torch.full_like(dev.q, float("nan"))
            launch(out)
            torch.cuda.synchronize()
            outs.append(out_to_f64(out))
        g_out = torch.full_like(dev.q, float("nan"))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch(g_out)
        for rep in range(3):
            g_out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            outs.append(out_to_f64(g_out))
        for i, o in enumerate(outs):
            err = max_err(o, ref, q)
            say(f"    partition {ps} launch {i}: max-abs error {err:.3g}")
            assert err <= TOL[kv]
            assert np.array_equal(o, outs[0]), "launches differ"
        del g


# ------------------------------------------------------------------ moving maxima
# Scores that rise along the context, fall, or jump at scattered positions:
# the running maximum of the online softmax moves (or stays) in every way the
# kernels distinguish — moved by more or less than their slack, at chunk
# starts or inside chunks, in single-pass, balanced and partitioned launches.
DRIFT = [
    # kv, q, H, Hkv
    ("bf16", "bf16", 8, 1),
    ("f16", "f16", 8, 1),
    ("fp8_e4m3", "f16", 8, 1),
    ("f16", "f16", 2, 2),
    ("fp8_e4m3", "f16", 71, 1),
]


@pytest.mark.parametrize("drift", ["rising", "falling", "spikes"])
@pytest.mark.parametrize("kv,q,H,Hkv", DRIFT)
def test_score_drift(kv, q, H, Hkv, drift):
    ctx = [1, 15, 16, 17, 300, 700]
    case = W.make_decode_case(f"drift_{drift}_{kv}_{H}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=128 if H <= 8 else 64, block_size=16,
                              context_lens=ctx, kv_dtype=kv, q_dtype=q, spare_blocks=3,
                              salt=H, key_drift=drift)
    run_and_check(case, partitions=(0, -1, 64))


# ------------------------------------------------------------------ shared prompts
# Tables in which sequences reference their predecessor's first blocks (the
# parallel samples of one prompt after a fork), in every launch mode: runs of
# sharing sequences of several lengths, sharing that breaks off along a run,
# long shared prefixes, small and large blocks, sequences cut across workers
# of the balanced split, runs across the schedule's 1024-sequence windows.
# The oracle reads every sequence through its own table.
def _share(case, groups):
    """groups: (first sequence, sequences, shared blocks) — the later sequences'
    first table entries are made the first one's."""
    t = case.block_tables
    bs = case.block_size
    for lead, n, k in groups:
        for j in range(lead + 1, lead + n):
            assert k * bs <= min(case.context_lens[j], case.context_lens[lead])
            t[j, :k] = t[lead, :k]
    return case


SHARE_CASES = [
    # name, kv, q, D, bs, H, Hkv, ctx, groups (first, sequences, shared blocks)
    ("g8_pairs", "bf16", "bf16", 128, 16, 64, 8,
     [521, 530, 600, 512, 300, 330, 400, 321, 90, 1, 17, 700],
     [(0, 4, 32), (5, 3, 20)]),
    ("g4_six_empty_tail", "f16", "f16", 128, 32, 16, 4,
     [320, 321, 350, 370, 330, 400, 5], [(0, 6, 10)]),
    ("g2_nine_fp8", "fp8_e4m3", "f16", 64, 8, 4, 2,
     [330, 331, 340, 360, 333, 350, 420, 336, 400, 44], [(0, 9, 40)]),
    ("g8_broken_chain", "bf16", "bf16", 128, 16, 16, 2,
     [400, 410, 420, 430, 300, 500], [(0, 2, 20), (1, 2, 10), (2, 2, 18), (4, 2, 16)]),
    ("g4_long_prefix", "f16", "f16", 64, 16, 8, 2,
     [2500, 2410, 1030, 1040, 1024, 1050, 1100, 1045], [(0, 2, 150), (2, 2, 64), (4, 2, 64), (6, 2, 65)]),
    ("g8_bs64_and_bs4", "bf16", "bf16", 128, 64, 16, 2, [600, 640, 700, 20], [(0, 3, 9)]),
    ("g4_bs4", "f16", "f16", 128, 4, 8, 2, [270, 290, 300, 260, 3], [(0, 4, 65)]),
    ("g8_fp8_q_bf16", "fp8_e4m3", "bf16", 128, 16, 16, 2, [700, 720, 650, 2], [(0, 3, 40)]),
]


@pytest.mark.parametrize("name,kv,q,D,bs,H,Hkv,ctx,groups", SHARE_CASES,
                         ids=[c[0] for c in SHARE_CASES])
def test_shared_prompt_groups(name, kv, q, D, bs, H, Hkv, ctx, groups):
    case = W.make_decode_case(f"share_{name}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=D, block_size=bs, context_lens=ctx,
                              kv_dtype=kv, q_dtype=q, spare_blocks=5, append=False, salt=len(name))
    run_and_check(_share(case, groups), partitions=(-1, 0, 64))


def test_shared_prompt_groups_cut_across_workers():
    """Enough work that balanced ranges are a few hundred tokens, so sharing
    sequences are cut across several workers and merged."""
    rng = np.random.default_rng(11)
    ctx, groups = [], []
    for g in range(12):
        lead = len(ctx)
        shared = int(rng.integers(20, 60))
        n = int(rng.integers(2, 6))
        ctx += [shared * 16 + int(rng.integers(0, 300)) for _ in range(n)]
        groups.append((lead, n, shared))
        ctx.append(int(rng.integers(1, 1500)))             # an unrelated sequence between groups
    case = W.make_decode_case("share_cut", "tiny", num_seqs=len(ctx), num_heads=64, num_kv_heads=8,
                              head_dim=128, block_size=16, context_lens=ctx, kv_dtype="bf16",
                              q_dtype="bf16", spare_blocks=5, append=False, salt=3)
    run_and_check(_share(case, groups), partitions=(-1, 0))


def test_shared_prompt_groups_at_window_edges():
    """Runs of sharing sequences across the schedule's 1024-sequence window boundary."""
    ctx = [int(x) for x in np.random.default_rng(5).integers(0, 40, size=1100)]
    for i in list(range(1018, 1030)) + [0, 1, 2, 1098, 1099]:
        ctx[i] = 300 + (i % 7) * 10
    case = W.make_decode_case("share_windows", "tiny", num_seqs=len(ctx), num_heads=8,
                              num_kv_heads=2, head_dim=64, block_size=16, context_lens=ctx,
                              kv_dtype="f16", q_dtype="f16", spare_blocks=5, append=False, salt=9)
    run_and_check(_share(case, [(1018, 12, 18), (0, 3, 17), (1098, 2, 16)]), partitions=(-1, 0))


# ------------------------------------------------------------------ item transitions
# Few tokens per worker, so every worker streams many items back to back, with
# empty contexts (items with no tokens) and one-chunk items between longer ones.
@pytest.mark.parametrize("kv,q,H,Hkv,bs", [("bf16", "bf16", 64, 8, 16), ("fp8_e4m3", "f16", 8, 4, 32),
                                           ("f16", "f16", 71, 1, 16), ("f16", "f16", 16, 2, 64)])
def test_item_transitions_with_empty_contexts(kv, q, H, Hkv, bs):
    ctx = [0, 5, 0, 0, 40, 0, 16, 17, 0, 300, 33, 0, 1, 64, 0, 0, 129, 2, 0, 31] * 3
    case = W.make_decode_case(f"transitions_{kv}_{H}_{bs}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=128 if H != 71 else 64, block_size=bs,
                              context_lens=ctx, kv_dtype=kv, q_dtype=q, spare_blocks=3, salt=bs + H)
    run_and_check(case, partitions=(-1, 0, 16))


# ------------------------------------------------------------------ seeded random configurations
def _random_config(seed):
    r = np.random.default_rng(1000 + seed)
    kv, q = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("fp8_e4m3", "f16"),
             ("fp8_e4m3", "bf16"), ("fp8_e4m3", "f32")][int(r.integers(0, 6))]
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 3, 4, 5, 8, 16, 20, 33, 71]))
    bs = int(r.choice([1, 2, 4, 8, 16, 32, 64, 128, 256]))
    S = int(r.integers(1, 24))
    mix = int(r.integers(0, 3))
    if mix == 0:                       # short and empty contexts
        ctx = r.integers(0, 40, size=S)
    elif mix == 1:                     # one long context among short ones
        ctx = r.integers(1, 200, size=S)
        ctx[int(r.integers(0, S))] = int(r.integers(1500, 5000))
    else:                              # log-normal
        ctx = np.clip(np.rint(np.exp(r.normal(np.log(300), 0.8, size=S))), 1, 3000)
    return kv, q, D, bs, G * Hkv, Hkv, [int(c) for c in ctx]


@pytest.mark.parametrize("seed", range(6))
def test_random_large_groups_many_sequences(seed):
    """The workgroup kernel (17-128 query heads per KV head) over batches of 100-600
    sequences: many workers, contexts cut across workers at every range boundary,
    items of every length, one or two workgroups per CU by head count."""
    r = np.random.default_rng(7000 + seed)
    kv, q = [("fp8_e4m3", "f16"), ("fp8_e4m3", "bf16"), ("f16", "f16"), ("bf16", "bf16")][seed % 4]
    D = [64, 128][(seed // 2) % 2] if kv != "fp8_e4m3" or seed % 3 else 64
    G = int(r.choice([17, 24, 40, 48, 64, 71, 100, 128]))
    Hkv = int(r.choice([1, 2]))
    bs = int(r.choice([8, 16, 32, 64]))
    S = int(r.integers(100, 600))
    ctx = (r.integers(1, 1500, size=S) if seed % 2 else
           np.clip(np.rint(np.exp(r.normal(np.log(300), 0.9, size=S))), 1, 3000)).astype(int)
    say(f"[case] large groups seed {seed}: {kv}/{q} D={D} G={G} Hkv={Hkv} bs={bs} S={S}")
    case = W.make_decode_case(f"large_group_{seed}", "tiny", num_seqs=S, num_heads=G * Hkv,
                              num_kv_heads=Hkv, head_dim=D, block_size=bs,
                              context_lens=[int(c) for c in ctx], kv_dtype=kv, q_dtype=q,
                              spare_blocks=9, salt=300 + seed)
    run_and_check(case, partitions=(-1, 512))


@pytest.mark.parametrize("seed", range(6))
def test_random_small_groups_many_sequences(seed):
    """The per-head (G = 1) and per-tile (2-16 heads per KV head) kernels over batches
    of 100-600 sequences: many workers (one per wavefront), every range boundary
    cutting a context."""
    r = np.random.default_rng(8000 + seed)
    kv, q = [("f16", "f16"), ("bf16", "bf16"), ("fp8_e4m3", "f16"), ("f32", "f32"),
             ("fp8_e4m3", "bf16"), ("f16", "f16")][seed]
    D = [64, 128][seed % 2]
    G = int(r.choice([1, 2, 4, 8, 16]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    bs = int(r.choice([8, 16, 32]))
    S = int(r.integers(100, 600))
    ctx = (r.integers(1, 1200, size=S) if seed % 2 else
           np.clip(np.rint(np.exp(r.normal(np.log(250), 0.9, size=S))), 1, 2500)).astype(int)
    say(f"[case] small groups seed {seed}: {kv}/{q} D={D} G={G} Hkv={Hkv} bs={bs} S={S}")
    case = W.make_decode_case(f"small_group_{seed}", "tiny", num_seqs=S, num_heads=G * Hkv,
                              num_kv_heads=Hkv, head_dim=D, block_size=bs,
                              context_lens=[int(c) for c in ctx], kv_dtype=kv, q_dtype=q,
                              spare_blocks=9, salt=400 + seed)
    run_and_check(case, partitions=(-1, 512))


@pytest.mark.parametrize("seed", range(48))
def test_random_configurations(seed):
    kv, q, D, bs, H, Hkv, ctx = _random_config(seed)
    case = W.make_decode_case(f"random_{seed}", "tiny", num_seqs=len(ctx), num_heads=H,
                              num_kv_heads=Hkv, head_dim=D, block_size=bs, context_lens=ctx,
                              kv_dtype=kv, q_dtype=q, spare_blocks=int(seed % 5), salt=seed,
                              max_blocks=int(W.blocks_needed(ctx, bs).max()) + 1 + seed % 3)
    run_and_check(case, partitions=(0, -1, max(bs, 64 // bs * bs), 512))
