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
