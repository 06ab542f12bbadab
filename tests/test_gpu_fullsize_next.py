"""GPU parity of the next rows at the sizes bench.py times them, in the same
launch configurations:

* sliding-window decode on the window batch (32 sequences of 4096 .. 16384
  positions, the Llama-3-8B layer shape, W = 4096), balanced split, single
  pass and fixed 512-position partitions, with every table entry of a block
  wholly before a sequence's window set to -1 and its contents NaN (released
  blocks: never read); every sequence compared with the oracle, every output
  checked finite;
* prefill on 16 whole prompts of 2048 positions and on 16 chunks of 512
  queries after cached prefixes of 0 .. 3584 positions (the same shape):
  every query row of the first sequence (the oracle's prefill of that whole
  sequence) and 90 more sampled across the others (first and last query,
  block edges, random others), each compared with the oracle on its own (a
  query at position p is a one-query prefill over positions 0 .. p through
  the same table), every output checked finite.

The inputs follow bench.py's recipe for those workloads (same seeds, same
generators).  Each ``MARGIN`` line records the measured error against its
bar.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_91_amd import pa
from paged_kv_cache_91_amd import workloads as W
from gpu_util import DEV, DeviceWorkload, max_err, out_f64, say, subset, to_dev, tol_for

pytestmark = pytest.mark.gpu

NAN_BF16 = np.uint16(0x7FC0)


def margin(name, part, rows, err, tol):
    say(f"MARGIN {name} partition={part} rows={rows} max_abs_err={err:.3e} tol={tol:g}")


def window_batch():
    rng = np.random.default_rng(9)
    lens = rng.integers(4096, 16385, size=32)
    need = int(sum(-(-int(n) // 16) for n in lens))
    return W.build_decode(9, name="window-4096-bf16", q_dtype="bf16", kv_dtype="bf16", num_q_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=16, num_blocks=need + 64,
                          context_lens=lens, rng=rng)


def test_window_decode_full():
    window = 4096
    wl = window_batch()
    bs = wl.block_size
    tables = wl.block_tables.copy()
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    for s, n in enumerate(wl.context_lens):
        lo = oracle.window_start(int(n), window)
        dead = tables[s, :lo // bs].copy()
        if len(dead):
            kp[dead] = NAN_BF16
            vp[dead] = NAN_BF16
            tables[s, :lo // bs] = -1
    seqs = list(range(wl.num_seqs))
    ref = np.stack([oracle.oracle_decode(sub.q, sub.q_dtype, sub.k_pool, sub.v_pool, sub.kv_dtype, sub.block_tables,
                                         sub.context_lens, sub.scale, window=window)[0]
                    for sub in (subset(wl, [s]) for s in seqs)])
    dev = DeviceWorkload(wl, tables=tables)
    dev.k_pool, dev.v_pool = to_dev(kp, "bf16"), to_dev(vp, "bf16")
    dev.pool = pa.make_pool(dev.k_pool, dev.v_pool, dtype="bf16")
    for part in (pa.PA_PARTITION_AUTO, 0, 512):
        out = torch.full_like(dev.q, float("nan"))
        got = out_f64(pa.pa_decode_window(dev.q, dev.pool, dev.tables, dev.ctx, window, wl.scale, out=out,
                                          partition_size=part, q_dtype="bf16"))
        assert np.isfinite(got).all(), part
        err = max_err(got[seqs], ref)
        margin("window-4096-bf16", part, f"{len(seqs)}seqs", err, tol_for(wl))
        assert err <= tol_for(wl), (part, err)


def prefill_inputs(kind):
    rng = np.random.default_rng(13)
    S = 16
    if kind == "prefill":
        lens = np.full(S, 2048)
        qlens = lens.copy()
    else:
        qlens = np.full(S, 512)
        lens = rng.integers(0, 3585, size=S) + qlens
    need = int(sum(-(-int(n) // 16) for n in lens))
    wl = W.build_decode(13, name=kind, q_dtype="bf16", kv_dtype="bf16", num_q_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16, num_blocks=need + 16, context_lens=lens, rng=rng)
    T = int(qlens.sum())
    q = W.cast_f32(W.normal_f32(13, 9, T * 32 * 128), "bf16").reshape(T, 32, 128)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return wl, q, qs


@pytest.mark.parametrize("kind", ["prefill", "prefill-chunk"])
def test_prefill_full(kind):
    wl, q, qs = prefill_inputs(kind)
    dev = DeviceWorkload(wl)
    qd = to_dev(q, "bf16")
    out = torch.full_like(qd, float("nan"))
    got = out_f64(pa.pa_prefill(qd, dev.pool, dev.tables, dev.ctx, torch.from_numpy(qs).to(DEV), wl.scale,
                                out=out, q_dtype="bf16"))
    assert np.isfinite(got).all()
    # the first sequence whole
    a0, b0 = int(qs[0]), int(qs[1])
    whole = oracle.oracle_prefill(q[a0:b0], "bf16", wl.k_pool, wl.v_pool, "bf16", wl.block_tables[:1],
                                  wl.context_lens[:1], np.array([0, b0 - a0]), wl.scale)
    errs = [max_err(got[a0:b0], whole)]
    # sampled rows of the others: per sequence its first and last query,
    # queries at block edges, and random others (90 in all)
    rng = np.random.default_rng(131)
    rows = []
    for s in range(1, len(wl.context_lens)):
        a, b = int(qs[s]), int(qs[s + 1])
        picks = {a, b - 1, min(b - 1, a + 15), min(b - 1, a + 16)} | set(int(x) for x in rng.integers(a, b, 2))
        rows += sorted(picks)[:6]
    for row in rows:
        s = int(np.searchsorted(qs, row, side="right") - 1)
        n, L = int(wl.context_lens[s]), int(qs[s + 1] - qs[s])
        p = n - L + (row - int(qs[s]))                # the query's position
        ref = oracle.oracle_prefill(q[row:row + 1], "bf16", wl.k_pool, wl.v_pool, "bf16", wl.block_tables[s:s + 1],
                                    np.array([p + 1]), np.array([0, 1]), wl.scale)
        errs.append(max_err(got[row:row + 1], ref))
    err = max(errs)
    margin(kind, "-", (b0 - a0) + len(rows), err, tol_for(wl))
    assert err <= tol_for(wl), err
