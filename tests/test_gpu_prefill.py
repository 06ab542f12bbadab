"""GPU parity of pa_prefill (causal multi-query attention over the paged
cache) against the float64 oracle's oracle_prefill: whole prompts and
chunks after a cached prefix, lengths straddling block edges, with and
without a sliding window, on the matrix-core kernel's shapes (head dim 128,
bf16/f16, block 16/32, groups 1, 2, 4, 8) and on the vector kernel's
(other groups, head dims, fp32, fp8 caches); unused pool memory is NaN, so
any read outside a sequence's positions shows up.  The last query of each
sequence must also match pa_decode's decode step."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_91_amd import pa
from paged_kv_cache_91_amd import workloads as W
from gpu_util import DEV, DeviceWorkload, max_err, out_f64, say, to_dev, tol_for

pytestmark = pytest.mark.gpu


def prefill_case(seed, qd, kd, hq, hkv, d, bs, lens, qlens):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens)
    need = sum(-(-int(n) // bs) for n in lens)
    if kd == "fp8_e4m3":
        wl = W.build_write_filled(seed, name="prefill-fp8", q_dtype=qd, src_dtype="bf16", kv_dtype=kd,
                                  num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                                  num_blocks=need + 4, context_lens=lens, rng=rng)
    else:
        wl = W.build_decode(seed, name="prefill", q_dtype=qd, kv_dtype=kd, num_q_heads=hq, num_kv_heads=hkv,
                            head_dim=d, block_size=bs, num_blocks=need + 4, context_lens=lens, rng=rng,
                            poison=True)
    T = int(sum(qlens))
    q = W.cast_f32(W.normal_f32(seed, 9, T * hq * d), qd).reshape(T, hq, d)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return wl, q, qs


def run_case(wl, q, qs, window=0):
    dev = DeviceWorkload(wl)
    kp, vp = wl.k_pool, wl.v_pool
    if wl.write_k is not None:
        dev.write()
        kp, vp = oracle.oracle_write(wl.write_k, wl.write_v, wl.write_src_dtype, wl.slot_mapping, kp, vp,
                                     wl.kv_dtype, wl.k_scale, wl.v_scale)
    ref = oracle.oracle_prefill(q, wl.q_dtype, kp, vp, wl.kv_dtype, wl.block_tables, wl.context_lens, qs,
                                wl.scale, wl.k_scale, wl.v_scale, window=window)
    qd = to_dev(q, wl.q_dtype)
    out = torch.full_like(qd, float("nan"))
    got = out_f64(pa.pa_prefill(qd, dev.pool, dev.tables, dev.ctx, torch.from_numpy(qs).to(DEV), wl.scale,
                                out=out, window=window, q_dtype=wl.q_dtype))
    return got, ref, dev, qd


SHAPES = [
    # (q_dtype, kv_dtype, Hq, Hkv, D, bs)
    ("bf16", "bf16", 32, 8, 128, 16),     # matrix cores, group 4 (the 8B layer shape)
    ("f16", "f16", 8, 8, 128, 16),        # group 1
    ("bf16", "bf16", 16, 8, 128, 32),     # group 2, block 32
    ("f16", "f16", 64, 8, 128, 32),       # group 8
    ("bf16", "bf16", 12, 4, 128, 16),     # group 3: vector kernel
    ("bf16", "bf16", 8, 2, 64, 8),        # head dim 64: vector kernel
    ("f32", "f32", 4, 2, 8, 4),
    ("bf16", "fp8_e4m3", 16, 4, 128, 32),  # fp8 cache: vector kernel
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
@pytest.mark.parametrize("window", [0, 50])
def test_prefill_shapes(shape, window):
    qd, kd, hq, hkv, d, bs = shape
    # whole prompts straddling block edges, then chunks after a cached prefix
    lens = [1, 15, 16, 17, 33, 100, 257, 300, 1000]
    qlens = [1, 15, 16, 17, 33, 100, 257, 64, 33]
    wl, q, qs = prefill_case(600 + hq + d + bs, qd, kd, hq, hkv, d, bs, lens, qlens)
    got, ref, _, _ = run_case(wl, q, qs, window)
    err = max_err(got, ref)
    say(f"[prefill] {shape} window {window}: rows {len(q)} max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= tol_for(wl), err


def test_prefill_long_chunk_and_many_sequences():
    """Chunks of 512 queries after prefixes of up to 1500 positions, and a
    batch past 64 sequences (the block lookup's second scan chunk)."""
    rng = np.random.default_rng(610)
    lens = list(rng.integers(513, 2000, size=6)) + list(rng.integers(1, 40, size=70))
    qlens = [512] * 6 + [int(min(n, rng.integers(1, 9))) for n in lens[6:]]
    wl, q, qs = prefill_case(611, "bf16", "bf16", 32, 8, 128, 16, lens, qlens)
    got, ref, _, _ = run_case(wl, q, qs)
    err = max_err(got, ref)
    say(f"[prefill] long chunks: rows {len(q)} max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= 2e-2


@pytest.mark.parametrize("shape", [("bf16", "bf16", 32, 8, 128, 16), ("f16", "f16", 40, 40, 128, 16)])
def test_prefill_last_query_is_the_decode_step(shape):
    qd, kd, hq, hkv, d, bs = shape
    lens = [5, 16, 17, 200, 701]
    qlens = [5, 3, 17, 64, 1]
    wl, q, qs = prefill_case(620, qd, kd, hq, hkv, d, bs, lens, qlens)
    got, ref, dev, qd_t = run_case(wl, q, qs)
    assert max_err(got, ref) <= 2e-2
    last = torch.from_numpy(qs[1:] - 1).to(DEV)
    dec = out_f64(pa.pa_decode(qd_t[last].contiguous(), dev.pool, dev.tables, dev.ctx, wl.scale,
                               partition_size=pa.PA_PARTITION_AUTO, q_dtype=wl.q_dtype))
    assert max_err(got[qs[1:] - 1], dec) <= 2e-2


def test_prefill_bad_length_gives_nan_rows():
    lens, qlens = [40, 60, 30], [10, 20, 5]
    wl, q, qs = prefill_case(630, "bf16", "bf16", 32, 8, 128, 16, lens, qlens)
    dev = DeviceWorkload(wl)
    ctx = wl.context_lens.copy()
    ctx[1] = 10                                   # fewer positions than queries
    dev.ctx = torch.from_numpy(ctx).to(DEV)
    qd = to_dev(q, "bf16")
    got = out_f64(pa.pa_prefill(qd, dev.pool, dev.tables, dev.ctx, torch.from_numpy(qs).to(DEV), wl.scale,
                                out=torch.zeros_like(qd)))
    ref = oracle.oracle_prefill(q, "bf16", wl.k_pool, wl.v_pool, "bf16", wl.block_tables, wl.context_lens, qs,
                                wl.scale)
    assert np.isnan(got[qs[1]:qs[2]]).all()
    keep = np.r_[qs[0]:qs[1], qs[2]:qs[3]]
    assert max_err(got[keep], ref[keep]) <= 2e-2


@pytest.mark.parametrize("scale", [-0.09, 0.0])
@pytest.mark.parametrize("shape", [("bf16", "bf16", 32, 8, 128, 16), ("f16", "f16", 16, 8, 128, 32),
                                   ("bf16", "bf16", 12, 4, 128, 16)])
def test_prefill_negative_and_zero_scale(shape, scale):
    """Any finite scale: a negative one reverses the softmax's preference
    (the matrix-core kernel moves its sign onto q), zero gives the plain mean
    of the attended V rows."""
    qd, kd, hq, hkv, d, bs = shape
    lens, qlens = [1, 40, 129, 300], [1, 40, 64, 33]
    wl, q, qs = prefill_case(640 + hq, qd, kd, hq, hkv, d, bs, lens, qlens)
    wl.scale = scale
    got, ref, _, _ = run_case(wl, q, qs, window=0)
    err = max_err(got, ref)
    say(f"[prefill] {shape} scale {scale}: max abs err {err:.3e}")
    assert np.isfinite(got).all() and err <= tol_for(wl), err


@pytest.mark.parametrize("shape", [("bf16", "bf16", 32, 8, 128, 16), ("bf16", "bf16", 12, 4, 128, 16)],
                         ids=["matrix-cores", "vector"])
@pytest.mark.parametrize("bad", ["past-end", "negative-start", "decreasing", "huge-last"])
def test_prefill_malformed_query_start_stays_inside_out(shape, bad):
    """A query_start that breaks its rules must not make the call write
    outside out's num_tokens rows: out is a view inside a larger buffer whose
    guard rows must keep their value.  Sequences the malformed entries do not
    touch still match the oracle; the matrix-core kernel gives NaN for the
    rows it can place of a sequence that leaves [0, num_tokens)."""
    qd, kd, hq, hkv, d, bs = shape
    lens, qlens = [40, 60, 50], [10, 20, 5]
    wl, q, qs = prefill_case(650 + hq, qd, kd, hq, hkv, d, bs, lens, qlens)
    T = len(q)
    bad_qs = {"past-end": [0, 10, 30, 45], "negative-start": [-8, 10, 30, 35],
              "decreasing": [0, 25, 10, 35], "huge-last": [0, 10, 30, 2**31 - 1]}[bad]
    clean = {"past-end": [0, 1], "negative-start": [1, 2], "decreasing": [], "huge-last": [0, 1]}[bad]
    dev = DeviceWorkload(wl)
    qd_t = to_dev(q, qd)
    guard = 64
    buf = torch.full((guard + T + guard, hq, d), 3.0, dtype=qd_t.dtype, device=DEV)
    out = buf[guard:guard + T]
    say(f"[prefill] malformed query_start {bad} {shape}")
    pa.pa_prefill(qd_t, dev.pool, dev.tables, dev.ctx, torch.tensor(bad_qs, dtype=torch.int32, device=DEV),
                  wl.scale, out=out)
    torch.cuda.synchronize()
    host = buf.float().cpu().numpy()
    assert (host[:guard] == 3.0).all() and (host[guard + T:] == 3.0).all()
    got = host[guard:guard + T].astype(np.float64)
    ref = oracle.oracle_prefill(q, qd, wl.k_pool, wl.v_pool, kd, wl.block_tables, wl.context_lens, qs, wl.scale)
    for s in clean:
        rows = slice(qs[s], qs[s + 1])
        assert max_err(got[rows], ref[rows]) <= tol_for(wl), (s, bad)
    if hq // hkv == 4 and bad in ("past-end", "negative-start"):
        s = 2 if bad == "past-end" else 0
        assert np.isnan(got[max(bad_qs[s], 0):min(bad_qs[s + 1], T)]).all()
