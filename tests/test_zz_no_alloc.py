"""pa_decode_noalloc (the library's static scratch instead of a caller's
workspace) against pa_decode with a workspace, through the C ABI: the same
kernels and the same work split, so the outputs must agree bit for bit, and
both must match the float64 oracle.  Each mode is called twice in a row, the
second time on a smaller batch, so the second call finds the scratch as the
first left it."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_91_amd import pa
from paged_kv_cache_91_amd import workloads as W
from gpu_util import DeviceWorkload, max_err, out_f64, say

pytestmark = pytest.mark.gpu


def _oracle(wl):
    return oracle.oracle_decode(wl.q, wl.q_dtype, wl.k_pool, wl.v_pool, wl.kv_dtype, wl.block_tables,
                                wl.context_lens, wl.scale, wl.k_scale, wl.v_scale)


def _both(dev, part):
    wl = dev.wl
    a = torch.full_like(dev.q, float("nan"))
    b = torch.full_like(dev.q, float("nan"))
    pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, out=a, partition_size=part,
                 q_dtype=wl.q_dtype)
    pa.pa_decode_noalloc(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, b, partition_size=part,
                         q_dtype=wl.q_dtype)
    torch.cuda.synchronize()
    return out_f64(a), out_f64(b)


BATCHES = [dict(seed=81, num_seqs=9, ctx_range=(1, 1500), num_blocks=900),
           dict(seed=82, num_seqs=3, ctx_range=(1, 300), num_blocks=64)]


@pytest.mark.parametrize("part", [pa.PA_PARTITION_AUTO, 64, 0])
def test_noalloc_matches_pa_decode_twice(part):
    for i, kw in enumerate(BATCHES):
        wl = W.config2(**kw)
        dev = DeviceWorkload(wl)
        with_ws, no_alloc = _both(dev, part)
        err = max_err(no_alloc, _oracle(wl))
        say(f"[noalloc] partition {part} call {i}: S={wl.num_seqs} max abs err {err:.3e}")
        assert np.isfinite(no_alloc).all()
        assert np.array_equal(no_alloc, with_ws), (part, i)
        assert err <= 2e-2


def test_noalloc_fp8_long_rows():
    rng = np.random.default_rng(83)
    lens = np.array([1, 31, 33, 700, 2100])
    need = sum(-(-int(n) // 32) for n in lens)
    wl = W.build_write_filled(83, name="noalloc-fp8", q_dtype="bf16", src_dtype="bf16", kv_dtype="fp8_e4m3",
                              num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=32,
                              num_blocks=need + 3, context_lens=lens, rng=rng)
    dev = DeviceWorkload(wl)
    dev.write()
    kp, vp = oracle.oracle_write(wl.write_k, wl.write_v, wl.write_src_dtype, wl.slot_mapping, wl.k_pool,
                                 wl.v_pool, wl.kv_dtype, wl.k_scale, wl.v_scale)
    ref = oracle.oracle_decode(wl.q, wl.q_dtype, kp, vp, wl.kv_dtype, wl.block_tables, wl.context_lens,
                               wl.scale, wl.k_scale, wl.v_scale)
    for part in (pa.PA_PARTITION_AUTO, 512):
        with_ws, no_alloc = _both(dev, part)
        assert np.array_equal(no_alloc, with_ws), part
        assert max_err(no_alloc, ref) <= 6e-2


def test_noalloc_starts_clean_after_a_marked_call():
    """A call whose in-workgroup waits are forced to give up marks the static
    scratch; the next call clears the counters first and is exact again."""
    wl = W.config2(seed=84, num_seqs=8, ctx_range=(300, 1200), num_blocks=700)
    dev = DeviceWorkload(wl)
    ref = _oracle(wl)
    out = torch.full_like(dev.q, float("nan"))
    pa.pa_set_wait_polls(1)
    try:
        pa.pa_decode_noalloc(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, out,
                             partition_size=pa.PA_PARTITION_AUTO)
    finally:
        pa.pa_set_wait_polls(0)
    torch.cuda.synchronize()
    assert np.isnan(out_f64(out)).any()
    for _ in range(2):
        out = torch.full_like(dev.q, float("nan"))
        pa.pa_decode_noalloc(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, out,
                             partition_size=pa.PA_PARTITION_AUTO)
        assert max_err(out_f64(out), ref) <= 2e-2


def test_noalloc_rejects_a_split_beyond_the_scratch():
    """Fixed partitions of bs 16 over 2048-position tables for 2000
    sequences need about 1 GB of partials: refused, nothing enqueued."""
    s, hq, hkv, d, bs, maxb = 2000, 32, 8, 128, 16, 128
    need = pa.pa_decode_workspace_bytes(s, hq, hkv, d, maxb, bs, 16)
    assert need > pa.PA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((s, hq, d), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((8, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    pool = pa.make_pool(kp, vp)
    tables = torch.zeros((s, maxb), dtype=torch.int32, device="cuda")
    ctx = torch.ones((s,), dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(pa.PaError) as exc:
        pa.pa_decode_noalloc(q, pool, tables, ctx, 0.1, out, partition_size=16)
    assert exc.value.status == -3 and "static scratch" in str(exc.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
