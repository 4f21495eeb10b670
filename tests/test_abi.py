"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any device work
(these calls never reach the GPU)."""
import ctypes
import json
import os
import re

import pytest

import paged_kv_cache_129_amd as pa
from paged_kv_cache_129_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_worked_examples.json"),
                        encoding="utf-8"))

FAKE = ctypes.c_void_p(0x1000)        # never dereferenced: every call below fails validation
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 19
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == {s[0] for s in pa._SIGNATURES}


def test_version_and_status_strings():
    assert "gfx950" in pa.version()
    for code, name in pa.STATUS.items():
        assert lib.pa_status_string(code)
    assert lib.pa_status_string(-3).decode() == "Out of KV cache blocks"
    assert lib.pa_status_string(12345).decode() == "unknown status"


@pytest.mark.parametrize("row", GOLDEN["kv_bytes_per_token"], ids=lambda r: r["model"])
def test_kv_bytes_per_token(row):
    assert pa.kv_bytes_per_token(row["num_kv_heads"], row["head_dim"], row["num_layers"], "f16") \
        == row["bytes"]


def test_kv_bytes_per_token_fp8_and_errors():
    assert pa.kv_bytes_per_token(1, 64, 32, "fp8_e4m3") == 4096
    assert lib.pa_kv_bytes_per_token(0, 64, 32, 1) == -1
    assert lib.pa_kv_bytes_per_token(1, 64, 32, 7) == -1


def decode_call(**kw):
    args = dict(out=FAKE, q=FAKE, q_dtype=1, k_pool=FAKE, v_pool=FAKE, kv_dtype=1, tables=FAKE,
                max_blocks=4, ctx=FAKE, max_ctx=64, S=2, H=4, Hkv=2, D=128, bs=16, NB=8,
                scale=0.1, k_scale=1.0, v_scale=1.0, part=0, ws=NULL, ws_bytes=0, stream=NULL)
    args.update(kw)
    return lib.pa_paged_attention_decode(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(H=5, Hkv=2), -1),                 # heads not a multiple of kv heads
    (dict(bs=12), -1),                      # block size not a power of two
    (dict(bs=512), -1),
    (dict(D=96), -2),                       # unsupported head_dim
    (dict(q_dtype=0, kv_dtype=1), -2),      # q f32 with f16 cache
    (dict(q_dtype=3, kv_dtype=3), -2),      # fp8 query
    (dict(q_dtype=9), -1),
    (dict(kv_dtype=3, k_scale=0.0), -1),    # fp8 needs positive scales
    (dict(kv_dtype=3, v_scale=float("nan")), -1),
    (dict(scale=float("inf")), -1),
    (dict(out=NULL), -1),
    (dict(tables=NULL), -1),
    (dict(q=ctypes.c_void_p(0x1004)), -1),  # misaligned
    (dict(S=-1), -1),
    (dict(NB=0), -1),
    (dict(max_blocks=0), -1),
    (dict(part=-16), -1),
    (dict(part=16), -8),                    # split needs a workspace
    (dict(part=-1), -8),                    # so does the balanced split
    (dict(part=-1, ws=ctypes.c_void_p(0x1010), ws_bytes=1 << 30), -8),   # misaligned
    (dict(part=-2), -1),                    # -1 is the only negative partition size
    (dict(part=16, ws=ctypes.c_void_p(0x1000), ws_bytes=10), -8),
])
def test_decode_validation(kw, status):
    assert decode_call(**kw) == status


def test_decode_zero_sequences_is_noop():
    assert decode_call(S=0, out=NULL, q=NULL) == 0


def test_workspace_size():
    def r256(b):
        return (b + 255) // 256 * 256
    ws = pa.paged_attention_workspace_size
    # single pass, or every sequence within one partition: nothing
    assert ws(4, 8, 8, 128, 100, 0) == 0
    assert ws(4, 8, 8, 128, 512, 512) == 0
    # split-context: (max, sum, output) per (sequence, head, partition)
    assert ws(4, 8, 8, 128, 1025, 512) == r256(4 * 8 * 3 * 130 * 4)
    # balanced: two records per worker for each head of a work unit, then one
    # 6-word range descriptor per worker (at most 32 workers per CU), all per
    # started window of 1024 sequences (MI355X: 256 CUs, also the fallback
    # without a device).  A unit is one head (per-head kernel, up to 32 workers
    # per CU) or, for 2 <= G <= 128, all G heads of a KV head (matrix-core
    # kernels: up to 8 workers per CU for G <= 16, 4 beyond); the records are
    # sized for whichever needs more.
    cus = 256
    for S, H, Hkv, D, G in ((4, 8, 2, 128, 4), (4, 32, 32, 64, 1), (1500, 71, 1, 64, 71),
                            (4, 128, 1, 64, 128), (4, 100, 1, 128, 100), (4, 20, 1, 128, 20),
                            (4, 48, 1, 64, 48), (4, 17, 1, 64, 17), (4, 64, 8, 128, 8)):
        windows = (S + 1023) // 1024
        slots_per_cu = max(32, (4 if G > 16 else 8) * G) if G >= 2 else 32
        expect = r256(windows * cus * slots_per_cu * 2 * (D + 2) * 4) + \
            r256(windows * cus * 32 * 6 * 8)
        assert ws(S, H, Hkv, D, 100, -1) == expect, (S, H, Hkv, D)
    assert ws(0, 8, 8, 128, 100, 0) == 0
    assert ws(4, 8, 8, 128, 100, -2) == 0


def write_call(**kw):
    args = dict(k_new=FAKE, v_new=FAKE, src=1, k_pool=FAKE, v_pool=FAKE, kv=1, slots=FAKE, T=3,
                Hkv=2, D=64, bs=16, NB=8, ks=1.0, vs=1.0, stream=NULL)
    args.update(kw)
    return lib.pa_kv_cache_write(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(src=0, kv=1), -2), (dict(src=3, kv=1), -2), (dict(src=1, kv=3, ks=-1.0), -1),
    (dict(bs=3), -1), (dict(D=80), -2), (dict(T=-1), -1), (dict(slots=NULL), -1),
    (dict(k_pool=ctypes.c_void_p(0x1008)), -1), (dict(NB=0), -1), (dict(src=8), -1),
])
def test_write_validation(kw, status):
    assert write_call(**kw) == status


def test_write_zero_tokens_is_noop():
    assert write_call(T=0, k_new=NULL) == 0


def copy_call(**kw):
    """pa_copy_blocks with fake device addresses: only calls that the host-side
    checks reject (or that are no-ops) are made, so nothing is launched."""
    kp = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    vp = (ctypes.c_void_p * 2)(0x3000, 0x4000)
    args = dict(k=kp, v=vp, L=2, dt=1, Hkv=2, D=64, bs=16, NB=8, pairs=ctypes.c_void_p(0x5000),
                n=1, stream=NULL)
    args.update(kw)
    return lib.pa_copy_blocks(*args.values())


@pytest.mark.parametrize("kw", [dict(pairs=NULL), dict(pairs=ctypes.c_void_p(0x5004)), dict(n=-1),
                                dict(NB=0), dict(bs=12), dict(L=-1), dict(dt=7)])
def test_copy_validation(kw):
    assert copy_call(**kw) == -1


def test_copy_noop_and_null_pool():
    assert copy_call(n=0) == 0
    assert copy_call(L=0) == 0
    kp = (ctypes.c_void_p * 2)(0x1000, 0)
    assert copy_call(k=kp) == -1
    kp = (ctypes.c_void_p * 2)(0x1000, 0x2008)          # pool not 16-byte aligned
    assert copy_call(k=kp) == -1


# ------------------------------------------------------------------ binding checks (host only)
def _binding_tensors(kv_v_dtype, device_v="cpu"):
    import torch
    q = torch.zeros(2, 4, 64, dtype=torch.float16)
    kp = torch.zeros(8, 2, 16, 64, dtype=torch.float16)
    vp = torch.zeros(8, 2, 16, 64, dtype=kv_v_dtype, device=device_v)
    tables = torch.zeros(2, 4, dtype=torch.int32)
    ctx = torch.ones(2, dtype=torch.int32)
    return q, kp, vp, tables, ctx


def test_binding_rejects_kv_pools_of_different_dtypes():
    """A V pool of a narrower type than K's would be read past its end."""
    import torch
    q, kp, vp, tables, ctx = _binding_tensors(torch.uint8)
    with pytest.raises(ValueError, match="differ in dtype"):
        pa.paged_attention_decode(torch.empty_like(q), q, kp, vp, tables, ctx,
                                  max_context_len=64, scale=0.125)
    k_new = torch.zeros(2, 2, 64, dtype=torch.float16)
    slots = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError, match="differ in dtype"):
        pa.kv_cache_write(k_new, k_new.to(torch.bfloat16), kp, kp.clone(), slots)
    with pytest.raises(ValueError, match="differ in dtype"):
        pa.kv_cache_write(k_new, k_new, kp, vp, slots)


def test_binding_rejects_tensors_on_different_devices():
    import torch
    q, kp, vp, tables, ctx = _binding_tensors(torch.float16, device_v="meta")
    with pytest.raises(ValueError, match="different devices"):
        pa.paged_attention_decode(torch.empty_like(q), q, kp, vp, tables, ctx,
                                  max_context_len=64, scale=0.125)
    with pytest.raises(ValueError, match="different devices"):
        pa.copy_blocks([kp], [vp], [(0, 1)])


def test_binding_rejects_host_tensors():
    import torch
    q, kp, vp, tables, ctx = _binding_tensors(torch.float16)
    with pytest.raises(ValueError, match="device tensor"):
        pa.paged_attention_decode(torch.empty_like(q), q, kp, vp, tables, ctx,
                                  max_context_len=64, scale=0.125)


def test_stream_read_rejects_bad_arguments():
    # each of these fails validation before anything reaches the device
    assert lib.pa_stream_read(NULL, 16, FAKE, NULL) == -1
    assert lib.pa_stream_read(FAKE, 16, NULL, NULL) == -1
    assert lib.pa_stream_read(FAKE, 0, FAKE, NULL) == -1
    assert lib.pa_stream_read(FAKE, 24, FAKE, NULL) == -1
    assert lib.pa_stream_read(ctypes.c_void_p(0x1008), 16, FAKE, NULL) == -1
    assert lib.pa_stream_read(FAKE, 16, ctypes.c_void_p(0x1002), NULL) == -1
