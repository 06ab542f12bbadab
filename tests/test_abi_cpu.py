"""The C ABI without a GPU: libpa.so loads, exports every function
include/pa.h declares, and rejects bad arguments on the host before any
launch.  Only calls that fail validation (or enqueue nothing) are made."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_91_amd import pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

FAKE = 0x10000   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pa.lib()
    names = declared_functions()
    assert set(names) == set(pa.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = pa.lib()
    assert [lib.pa_status_string(s).decode() for s in (0, -1, -2, -3, -4, 7)] == [
        "PA_OK", "PA_ERR_INVALID_ARG", "PA_ERR_UNSUPPORTED", "PA_ERR_WORKSPACE", "PA_ERR_HIP",
        "PA_ERR_UNKNOWN"]
    assert lib.pa_version() >= 100


def test_workspace_bytes():
    # fixed partitions -- counters: 8 bytes per (sequence, head group), padded
    # to 256 bytes; partials: per (sequence, head group, partition, head slot)
    # m, l and D outputs
    assert pa.pa_decode_workspace_bytes(32, 64, 8, 128, 1024, 32, 512) == 2048 + 32 * 8 * 64 * 8 * 130 * 4
    assert pa.pa_decode_workspace_bytes(3, 2, 1, 8, 5, 4, 8) == 256 + 3 * 3 * 2 * 10 * 4
    # group 3 is handled as 4 head slots; group 16 as two head groups of 8
    assert pa.pa_decode_workspace_bytes(2, 12, 4, 64, 4, 16, 32) == 256 + 2 * 4 * 2 * 4 * 66 * 4
    assert pa.pa_decode_workspace_bytes(100, 32, 2, 64, 1, 16, 16) == 3328 + 100 * 2 * 2 * 1 * 8 * 66 * 4
    assert pa.pa_decode_workspace_bytes(3, 2, 1, 8, 5, 4, 0) == 0
    assert pa.pa_decode_workspace_bytes(0, 2, 1, 8, 5, 4, 8) == 0
    assert pa.pa_decode_workspace_bytes(3, 3, 2, 8, 5, 4, 8) == 0      # heads not a multiple
    # balanced split: 4 KiB of control words, a 128-byte counter line per
    # (sequence, head group), and two partial slots per range of each of the
    # 8 XCD shares, one range per streaming wave: 4 per compute unit (256
    # compute units and 8 XCDs assumed when no GPU can be queried, as here);
    # a slot holds D outputs per head and a 128-byte line of (m, l) pairs
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 128, 16, pa.PA_PARTITION_AUTO) == \
        4096 + 512 * 128 + 8 * 128 * 2 * (4 * 128 + 32) * 4
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 128, 16, -2) == 0


def _pool(**kw):
    base = dict(k_pool=FAKE, v_pool=FAKE * 2, num_blocks=16, num_kv_heads=2, block_size=16,
                head_dim=128, dtype=pa.PA_BF16, k_scale=1.0, v_scale=1.0)
    base.update(kw)
    return pa.KvPool(**base)


def _decode(pool, **kw):
    args = dict(q=FAKE * 3, q_dtype=pa.PA_BF16, num_seqs=2, num_q_heads=8, tables=FAKE * 4,
                maxb=4, ctx=FAKE * 5, scale=0.1, out=FAKE * 6, part=0, ws=None, ws_bytes=0)
    args.update(kw)
    return pa.lib().pa_decode(args["q"], args["q_dtype"], args["num_seqs"], args["num_q_heads"],
                              ctypes.byref(pool) if pool is not None else None, args["tables"],
                              args["maxb"], args["ctx"], args["scale"], args["out"], args["part"],
                              args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("pool_kw,expect", [
    (dict(block_size=3), -1),
    (dict(block_size=1), -1),
    (dict(block_size=512), -1),
    (dict(head_dim=96), -2),
    (dict(num_blocks=0), -1),
    (dict(num_kv_heads=0), -1),
    (dict(dtype=9), -1),
    (dict(k_pool=0), -1),
    (dict(v_pool=FAKE), -1),                       # aliases k_pool
    (dict(dtype=pa.PA_FP8_E4M3, k_scale=0.0), -1),
    (dict(dtype=pa.PA_FP8_E4M3, v_scale=float("inf")), -1),
    (dict(k_scale=2.0), -1),                       # scale on a bf16 pool
])
def test_decode_rejects_bad_pool(pool_kw, expect):
    assert _decode(_pool(**pool_kw)) == expect
    assert pa.lib().pa_last_error().decode()


@pytest.mark.parametrize("kw,expect", [
    (dict(num_q_heads=7), -1),                     # not a multiple of Hkv
    (dict(num_q_heads=0), -1),
    (dict(num_seqs=-1), -1),
    (dict(num_seqs=70000), -1),
    (dict(q=0), -1),
    (dict(out=FAKE * 3), -1),                      # aliases q
    (dict(maxb=0), -1),
    (dict(scale=float("nan")), -1),
    (dict(q_dtype=pa.PA_FP8_E4M3), -1),
    (dict(q_dtype=pa.PA_F16), -2),                 # f16 q with a bf16 pool
    (dict(part=24), -1),                           # not a multiple of block_size
    (dict(part=-16), -1),
    (dict(part=-1), -3),                           # balanced split needs a workspace
    (dict(part=32), -3),                           # no workspace
    (dict(part=32, ws=FAKE * 7, ws_bytes=16), -3), # too small
])
def test_decode_rejects_bad_args(kw, expect):
    assert _decode(_pool(), **kw) == expect


def test_decode_null_pool_and_empty_batch():
    assert _decode(None) == -1
    assert _decode(_pool(), num_seqs=0) == 0       # nothing to do: no launch


def test_write_and_copy_validation():
    lib = pa.lib()
    p = _pool()
    assert lib.pa_write_kv(FAKE, FAKE, pa.PA_BF16, -1, FAKE, ctypes.byref(p), None) == -1
    assert lib.pa_write_kv(FAKE, FAKE, pa.PA_BF16, 0, FAKE, ctypes.byref(p), None) == 0
    assert lib.pa_write_kv(0, FAKE, pa.PA_BF16, 4, FAKE, ctypes.byref(p), None) == -1
    assert lib.pa_write_kv(FAKE, FAKE, pa.PA_F16, 4, FAKE, ctypes.byref(p), None) == -2
    assert lib.pa_write_kv(FAKE, FAKE, 11, 4, FAKE, ctypes.byref(p), None) == -1
    fp8 = _pool(dtype=pa.PA_FP8_E4M3, k_scale=0.5, v_scale=0.25)
    assert lib.pa_write_kv(FAKE, FAKE, pa.PA_FP8_E4M3 + 5, 4, FAKE, ctypes.byref(fp8), None) == -1
    assert lib.pa_copy_blocks(ctypes.byref(p), FAKE, -1, None) == -1
    assert lib.pa_copy_blocks(ctypes.byref(p), FAKE, 0, None) == 0
    assert lib.pa_copy_blocks(ctypes.byref(p), None, 3, None) == -1
    assert lib.pa_copy_blocks(None, FAKE, 3, None) == -1


def test_time_next_decode_validation():
    lib = pa.lib()
    assert lib.pa_time_next_decode(FAKE, None) == -1
    assert lib.pa_time_next_decode(None, FAKE) == -1
    assert lib.pa_time_next_decode(None, None) == 0
    # a pair set and then consumed by a call that fails validation is gone
    assert lib.pa_time_next_decode(FAKE, FAKE * 2) == 0
    assert _decode(_pool(block_size=3)) == -1
    assert _decode(_pool(), num_seqs=0) == 0


def test_status_query_and_wait_polls_validation():
    lib = pa.lib()
    assert lib.pa_decode_status(FAKE, 8192, -1, None, None) == -1           # no status pointer
    assert lib.pa_decode_status(FAKE, 8192, -5, FAKE, None) == -1           # bad mode
    assert lib.pa_decode_status(FAKE, 100, -1, FAKE, None) == -3            # not a balanced-split workspace
    assert lib.pa_decode_status(None, 8192, -1, FAKE, None) == -3
    assert lib.pa_set_wait_polls(-1) == -1
    assert lib.pa_set_wait_polls(5) == 0
    assert lib.pa_set_wait_polls(0) == 0                                    # back to the default


def test_noalloc_validation_without_gpu():
    """Calls of pa_decode_noalloc that fail before touching the GPU."""
    lib = pa.lib()
    p = _pool()
    args = lambda **kw: dict(dict(q=FAKE, qd=pa.PA_BF16, s=4, hq=8, pool=ctypes.byref(p), bt=FAKE, maxb=8,
                                  ctx=FAKE, scale=0.1, out=FAKE * 2, part=0, stream=None), **kw)
    call = lambda a: lib.pa_decode_noalloc(a["q"], a["qd"], a["s"], a["hq"], a["pool"], a["bt"], a["maxb"],
                                           a["ctx"], a["scale"], a["out"], a["part"], a["stream"])
    assert call(args(pool=None)) == -1
    assert call(args(q=None)) == -1
    assert call(args(s=0)) == 0
    # a fixed-partition split far beyond the static scratch
    assert call(args(s=60000, maxb=4096, part=16)) == -3
    assert b"static scratch" in lib.pa_last_error()
