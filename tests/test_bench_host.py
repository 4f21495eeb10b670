"""CPU checks of bench.py's host logic: algorithmic byte counts against their
closed forms, the lookup of counter-measured traffic (same workload, launch
mode and block size, unchanged kernel sources only), and the one-GPU guard."""
import hashlib
import os
import subprocess
import sys

import numpy as np

import bench


def test_llama7b_layer_bytes_closed_form():
    # 64 sequences x 4096 tokens x K and V x 32 heads x 128 x fp16, plus q and out,
    # the 256 table entries of each sequence and the lengths
    ctx = np.full(64, 4096)
    assert bench.attention_bytes(ctx, 64, 32, 32, 128, 2, 2, 16) == \
        4_294_967_296 + 1_048_576 + 65_536 + 256 == 4_296_081_664
    # the write: every new token's K and V read (fp16) and stored (fp16), and its slot
    assert bench.write_bytes(64, 32, 128, 2, 2) == 2_097_664


def test_shared_prompt_blocks_counted_once():
    ctx = np.array([521, 521, 300])
    unique = int(ctx.sum()) - 512           # the second sample's 32 shared blocks of 16
    got = bench.attention_bytes(ctx, 3, 64, 8, 128, 2, 2, 16, unique_tokens=unique)
    want = unique * 2 * 8 * 128 * 2 + 2 * 3 * 64 * 128 * 2 + (33 + 33 + 19) * 4 + 3 * 4
    assert got == want


def _traffic_file(root, workload, part, bs, sources):
    h = hashlib.sha256()
    for src in sources:
        h.update(open(os.path.join(root, src), "rb").read())
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"k_{workload}.traffic.txt"), "w") as f:
        f.write("# a comment line = ignored\n")
        f.write(f"workload = {workload}\npartition_size = {part}\nblock_size = {bs}\n")
        f.write("sources = " + " ".join(sources) + f"\nsource_sha256 = {h.hexdigest()}\n")
        f.write("traffic_bytes = 123456789\n")


def test_traffic_lookup(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    _traffic_file(str(tmp_path), "wl", -1, 16, ["k.hip"])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("wl", -1, 16) == (123456789, "k_wl.traffic.txt")
    # another launch mode, block size or workload: no figure
    assert bench.read_traffic("wl", 0, 16) == (None, None)
    assert bench.read_traffic("wl", -1, 8) == (None, None)
    assert bench.read_traffic("other", -1, 16) == (None, None)
    # a kernel source changed since the counters were taken: no figure
    src.write_text("// kernel, changed\n")
    assert bench.read_traffic("wl", -1, 16) == (None, None)
    # a source of the profiled build is gone: no figure
    src.unlink()
    assert bench.read_traffic("wl", -1, 16) == (None, None)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_allocator_study_against_closed_forms():
    """The allocator study's readouts against what the pages' arithmetic fixes:
    blocks of one token never hold an empty slot (utilisation 1); reserving the
    maximum of 2,048 tokens in a ~15,700-token cache admits at most 7 requests at
    once (KV 缓存与分页注意力 §04: 12 GB / 2,048 positions = 7 sequences);
    utilisation falls as blocks grow (§14) and paged blocks beat every
    reservation policy (§05, §07)."""
    import paged_kv_cache_129_amd as pa
    r = bench.allocator_study(pa)
    toy, big = r["toy_176_slots"], r["opt13b_15700_tokens"]
    assert toy["block_1"]["utilisation"] == 1.0
    u = [toy[f"block_{b}"]["utilisation"] for b in (1, 2, 4, 8, 16)]
    assert all(x > y for x, y in zip(u, u[1:]))
    assert toy["reserve_20"]["max_concurrent"] == 176 // 20
    assert big["reserve_max"]["max_concurrent"] == 15700 // 2048 == 7
    assert big["paged_block_16"]["utilisation"] > big["reserve_exact"]["utilisation"] > \
        big["reserve_pow2"]["utilisation"] > big["reserve_max"]["utilisation"]
    assert big["paged_block_16"]["mean_concurrent"] > big["reserve_exact"]["mean_concurrent"]


def test_paged_policy_readout_matches_the_oracle_model():
    """The study's paged readout comes from the library allocator's counts; the
    oracle's allocator model, driven through the same trace, gives the same."""
    import paged_kv_cache_129_amd as pa
    import oracle

    class ModelPaged(bench.Paged):
        def __init__(self, capacity, block_size):
            self.a, self.bs = oracle.Allocator(capacity // block_size, block_size), block_size

        def admit(self, rid, first_len, final_len):
            try:
                self.a.add_seq(rid, first_len)
                return True
            except oracle.OutOfBlocks:
                return False

        def grow_all(self, rids):
            try:
                if rids:
                    self.a.append_slots(rids)
                return True
            except oracle.OutOfBlocks:
                return False

    rng = np.random.default_rng(5)
    finals = rng.integers(1, 21, size=30).tolist()
    for bs in (1, 4, 16):
        lib = bench.serve_trace(bench.Paged(pa, 176, bs), [1] * 30, finals)
        mod = bench.serve_trace(ModelPaged(176, bs), [1] * 30, finals)
        assert lib == mod


def test_committed_traffic_figures_match_the_sources():
    """Every committed counter summary still describes the kernels as they are: its
    sources hash to the recorded value, so bench.py reports its figure."""
    import glob
    paths = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "*.traffic.txt")))
    assert paths
    for path in paths:
        kv = dict(line.split("=", 1) for line in open(path)
                  if "=" in line and not line.lstrip().startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        figure, name = bench.read_traffic(kv["workload"], int(kv["partition_size"]),
                                          int(kv.get("block_size", "0")))
        assert name == os.path.basename(path), path
        assert figure == int(float(kv["traffic_bytes"]))
