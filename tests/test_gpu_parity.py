"""GPU parity at oracle-friendly sizes: every decode specialisation, single
pass and split-KV, the cache write (bit-exact), the block copy (bit-exact),
relabelling invariance, determinism, NaN-poisoned unused memory, and the
edge cases (empty, one-position and maximal contexts; out-of-range table
entries, lengths and slots handled without faulting).

Each test compares the HIP library, called through its binding, against the
float64 oracle on the same seeded inputs: max-abs error within 1e-5 (fp32),
2e-2 (fp16 / bf16) or 6e-2 (fp8 cache); writes and copies byte for byte.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_91_amd import pa
from paged_kv_cache_91_amd import workloads as W
from gpu_util import DEV, DeviceWorkload, dev_to_host, max_err, out_f64, say, to_dev, tol_for

pytestmark = pytest.mark.gpu


def oracle_out(wl, tables=None, k_pool=None, v_pool=None):
    return oracle.oracle_decode(wl.q, wl.q_dtype, wl.k_pool if k_pool is None else k_pool,
                                wl.v_pool if v_pool is None else v_pool, wl.kv_dtype,
                                wl.block_tables if tables is None else tables, wl.context_lens,
                                wl.scale, wl.k_scale, wl.v_scale)


def oracle_written(wl):
    return oracle.oracle_write(wl.write_k, wl.write_v, wl.write_src_dtype, wl.slot_mapping,
                               wl.k_pool, wl.v_pool, wl.kv_dtype, wl.k_scale, wl.v_scale)


def check_decode(wl, parts=(0,), label=""):
    say(f"[decode] {wl.name} {label} S={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"D={wl.head_dim} bs={wl.block_size} parts={parts}")
    dev = DeviceWorkload(wl)
    kp, vp = wl.k_pool, wl.v_pool
    if wl.write_k is not None:          # the workload's cache write comes first, on both sides
        dev.write()
        kp, vp = oracle_written(wl)
    ref = oracle_out(wl, k_pool=kp, v_pool=vp)
    outs = []
    for p in parts:
        got = out_f64(dev.decode(partition_size=p))
        err = max_err(got, ref)
        say(f"    partition {p}: max abs err {err:.3e}")
        assert np.isfinite(got).all()
        assert err <= tol_for(wl), f"partition {p}: {err}"
        outs.append(got)
    return outs


# ---------------------------------------------------------------------------
# tiny fp32 and the pages' scalar case
# ---------------------------------------------------------------------------

def test_tiny_fp32():
    wl = W.config1()
    check_decode(wl, parts=(0, 4, 8, pa.PA_PARTITION_AUTO))
    pinned = W.config1()
    pinned.block_tables = np.array([[7, 2], [9, 0]], dtype=np.int32)   # zerocoder.ru example tables
    check_decode(pinned, parts=(0, 4), label="tables [7,2],[9]")


def test_scalar_case_exactly_three():
    """K = 0, q = 1, V rows 1..5 at block 4 over two placements: exactly 3."""
    bs, d = 4, 8
    for placement in ([4, 1], [0, 1], [2, 5]):
        kp = np.full((8, 1, bs, d), np.nan, np.float32)
        vp = np.full((8, 1, bs, d), np.nan, np.float32)
        for pos in range(5):
            kp[placement[pos // bs], 0, pos % bs, :] = 0.0
            vp[placement[pos // bs], 0, pos % bs, :] = pos + 1
        q = torch.ones((1, 1, d), dtype=torch.float32, device=DEV)
        kt, vt = torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV)
        pool = pa.make_pool(kt, vt)
        tables = torch.tensor([placement], dtype=torch.int32, device=DEV)
        ctx = torch.tensor([5], dtype=torch.int32, device=DEV)
        for part in (0, 4):
            out = pa.pa_decode(q, pool, tables, ctx, 1.0, out=torch.full_like(q, float("nan")),
                               partition_size=part)
            assert out.cpu().numpy().tolist() == [[[3.0] * d]], (placement, part)


# ---------------------------------------------------------------------------
# every decode specialisation at small sizes
# ---------------------------------------------------------------------------

SHAPES = [
    # (q_dtype, kv_dtype, Hq, Hkv, D, bs)
    ("bf16", "bf16", 32, 8, 128, 16),     # Llama-3-8B layer shape
    ("f16", "f16", 40, 40, 128, 16),      # 13B MHA shape
    ("bf16", "bf16", 8, 8, 64, 16),
    ("f16", "f16", 16, 2, 256, 8),        # group 8
    ("bf16", "bf16", 12, 4, 128, 32),     # group 3 (masked head)
    ("f16", "f16", 32, 2, 64, 4),         # group 16 (two head groups)
    ("f32", "f32", 4, 2, 128, 16),
    ("f32", "f32", 2, 1, 8, 2),
    ("bf16", "bf16", 2, 1, 8, 64),
    ("f32", "f32", 8, 4, 256, 16),
    ("bf16", "bf16", 16, 8, 128, 16),     # group 2: two heads per head-dim-128 workgroup
    ("bf16", "bf16", 32, 2, 128, 16),     # group 16: two head groups of 8 per KV head
    ("f16", "f16", 48, 2, 128, 32),       # group 24: three head groups of 8
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_shapes(shape):
    qd, kd, hq, hkv, d, bs = shape
    rng = np.random.default_rng(100 + hq + d + bs)
    lens = np.concatenate([[1, bs, bs + 1, 3 * bs - 1], rng.integers(1, 300, size=4)])
    need = sum(-(-int(n) // bs) for n in lens)
    wl = W.build_decode(100 + d, name=f"shape-{qd}", q_dtype=qd, kv_dtype=kd, num_q_heads=hq,
                        num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=need + 7,
                        context_lens=lens, rng=rng)
    check_decode(wl, parts=(0, bs, 4 * bs, 512 if 512 % bs == 0 else 8 * bs, pa.PA_PARTITION_AUTO))


@pytest.mark.parametrize("shape", [("bf16", "bf16", 32, 8, 128, 16), ("f16", "f16", 8, 8, 128, 16),
                                   ("bf16", "bf16", 64, 8, 128, 32)], ids=lambda s: "-".join(map(str, s)))
def test_fixed_split_merges_many_partitions(shape):
    """The fixed split's merge folds a sequence's partitions in rounds of 8
    per lane group (up to 8 groups): with one block per partition, lengths
    of 16 to 3030 positions give from 1 to ~190 partitions, covering one and
    several rounds, groups with no partition, and a last round only partly
    filled."""
    qd, kd, hq, hkv, d, bs = shape
    rng = np.random.default_rng(700 + hq + bs)
    lens = np.array([16, 17, 1024, 1025, 2049, 3030])
    need = sum(-(-int(n) // bs) for n in lens)
    wl = W.build_decode(700 + hq, name=f"many-parts-{qd}", q_dtype=qd, kv_dtype=kd, num_q_heads=hq,
                        num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=need + 3,
                        context_lens=lens, rng=rng)
    check_decode(wl, parts=(bs, 16 * bs, pa.PA_PARTITION_AUTO), label="many partitions")


@pytest.mark.parametrize("kv", ["f16", "bf16"])
def test_split_partials_hold_large_values(kv):
    """The fixed split keeps each partition's output as a mean of V rows in
    the query dtype.  With every V value made positive and multiplied by
    2^12 (both exact; f16 values then reach ~2e4), the outputs are exactly
    2^12 times those of the positive unscaled problem, so out / 2^12 must
    meet the usual bar against the oracle on that problem at every partition
    size.  A partial kept unnormalised (a weighted sum of up to P rows)
    would pass f16's largest finite value here."""
    rng = np.random.default_rng(880)
    lens = np.array([1, 16, 17, 255, 256, 1000, 2049])
    bs = 16
    need = sum(-(-int(n) // bs) for n in lens)
    wl = W.build_decode(880, name=f"large-v-{kv}", q_dtype=kv, kv_dtype=kv, num_q_heads=32,
                        num_kv_heads=8, head_dim=128, block_size=bs, num_blocks=need + 3,
                        context_lens=lens, rng=rng)
    mul = 4096.0
    if kv == "bf16":
        wl.v_pool = wl.v_pool & np.uint16(0x7FFF)
        ref = oracle_out(wl)
        widened = (wl.v_pool.astype(np.uint32) << 16).view(np.float32) * np.float32(mul)
        wl.v_pool = (widened.view(np.uint32) >> 16).astype(np.uint16)
    else:
        wl.v_pool = np.abs(wl.v_pool)
        ref = oracle_out(wl)
        wl.v_pool = wl.v_pool * np.float16(mul)
        assert np.isfinite(wl.v_pool).all()
    dev = DeviceWorkload(wl)
    for p in (0, bs, 4 * bs, 512, pa.PA_PARTITION_AUTO):
        got = out_f64(dev.decode(partition_size=p))
        assert np.isfinite(got).all(), f"partition {p}"
        err = max_err(got / mul, ref)
        say(f"    large V ({kv}) partition {p}: max abs err of out / 2^12 {err:.3e}")
        assert err <= tol_for(wl), f"partition {p}: {err}"


FP8_SHAPES = [
    ("bf16", "bf16", 64, 8, 128, 32),     # long-context fp8 layer shape
    ("bf16", "f32", 8, 2, 64, 16),
    ("f16", "f16", 4, 4, 128, 8),
    ("bf16", "bf16", 16, 2, 256, 16),
    ("f16", "f16", 16, 4, 128, 32),       # f16 queries on the matrix-core kernels, group 4
    ("f16", "f16", 8, 8, 128, 16),        # the same, one head per KV head
]


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_fp8_cache(shape):
    qd, src, hq, hkv, d, bs = shape
    rng = np.random.default_rng(200 + hq + d)
    lens = np.concatenate([[1, bs - 1, bs, 2 * bs + 3], rng.integers(1, 700, size=3)])
    need = sum(-(-int(n) // bs) for n in lens)
    wl = W.build_write_filled(200 + d, name="fp8", q_dtype=qd, src_dtype=src, kv_dtype="fp8_e4m3",
                              num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                              num_blocks=need + 5, context_lens=lens, rng=rng)
    check_decode(wl, parts=(0, bs, 4 * bs, 512 if 512 % bs == 0 else 8 * bs, pa.PA_PARTITION_AUTO))


def test_fp8_decode_every_code():
    """Decoding of every finite e4m3 code, seen through pa_decode.  With one
    position the output is that position's V row times v_scale exactly (every
    e4m3 value times 2 is a bf16 value), so sequence s whose V row holds codes
    128*s .. 128*s+127 must return the oracle table's values bit for bit."""
    bs, d = 16, 128
    table = oracle.e4m3_table()
    kp = np.zeros((2, 1, bs, d), np.uint8)
    vp = np.zeros((2, 1, bs, d), np.uint8)
    codes = np.arange(256, dtype=np.uint8).reshape(2, d)
    codes[np.isnan(table[codes])] = 0                  # the two NaN codes become +0
    vp[:, 0, 0, :] = codes
    wl = W.Workload(name="fp8-codes", q_dtype="bf16", kv_dtype="fp8_e4m3", num_q_heads=2,
                    num_kv_heads=1, head_dim=d, block_size=bs, num_blocks=2,
                    q=W.cast_f32(np.ones((2, 2, d), np.float32), "bf16"), k_pool=kp, v_pool=vp,
                    block_tables=np.array([[0], [1]], np.int32),
                    context_lens=np.array([1, 1], np.int32), scale=0.125, k_scale=0.5, v_scale=2.0)
    expect = table[codes] * 2.0
    for part in (0, 16):
        got = out_f64(DeviceWorkload(wl).decode(partition_size=part))
        for h in range(2):
            assert np.array_equal(got[:, h, :], expect), part


# ---------------------------------------------------------------------------
# cache write and block copy: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("src,dst,d,bs", [
    ("f16", "f16", 128, 16), ("bf16", "bf16", 64, 8), ("f32", "f32", 8, 4),
    ("bf16", "fp8_e4m3", 128, 32), ("f16", "fp8_e4m3", 64, 16), ("f32", "fp8_e4m3", 128, 16),
    ("bf16", "fp8_e4m3", 8, 4), ("fp8_e4m3", "fp8_e4m3", 8, 2),
])
def test_write_bitexact(src, dst, d, bs):
    say(f"[write] {src}->{dst} D={d} bs={bs}")
    rng = np.random.default_rng(300 + d + bs)
    lens = rng.integers(1, 90, size=6)
    need = sum(-(-int(n) // bs) for n in lens)
    if src == "fp8_e4m3":
        wl = W.build_write_filled(301, name="w", q_dtype="bf16", src_dtype="bf16", kv_dtype="fp8_e4m3",
                                  num_q_heads=4, num_kv_heads=2, head_dim=d, block_size=bs,
                                  num_blocks=need + 3, context_lens=lens, rng=rng)
        # fp8 -> fp8 copy of codes: source rows are codes the oracle encoded
        codes_k = oracle.e4m3_encode(W.bf16_bits_to_f32(wl.write_k) * np.float32(1 / wl.k_scale))
        codes_v = oracle.e4m3_encode(W.bf16_bits_to_f32(wl.write_v) * np.float32(1 / wl.v_scale))
        wl.write_k, wl.write_v, wl.write_src_dtype = codes_k, codes_v, "fp8_e4m3"
        wl.k_scale = wl.v_scale = 1.0
    else:
        wl = W.build_write_filled(302, name="w", q_dtype="bf16" if src != "f32" else "f32",
                                  src_dtype=src, kv_dtype=dst, num_q_heads=4, num_kv_heads=2,
                                  head_dim=d, block_size=bs, num_blocks=need + 3,
                                  context_lens=lens, rng=rng)
    # scale the rows so the fp8 encoder sees subnormals, ties and saturation
    if dst == "fp8_e4m3" and src != "fp8_e4m3":
        wl.k_scale = wl.k_scale * 0.75      # some |x / scale| > 448: saturates
    dev = DeviceWorkload(wl)
    dev.write()
    gk, gv = dev.pools_host()
    rk, rv = oracle_written(wl)
    assert np.array_equal(gk.view(np.uint8), rk.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), rv.view(np.uint8))


def test_write_skips_out_of_range_slots():
    wl = W.config3(num_seqs=4, num_blocks=256, length_cap=100)
    dev = DeviceWorkload(wl)
    before_k, _ = dev.pools_host()
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    slots[2] = wl.num_blocks * wl.block_size          # one past the end
    k = to_dev(wl.write_k, "f16")
    v = to_dev(wl.write_v, "f16")
    pa.pa_write_kv(k, v, torch.from_numpy(slots).to(DEV), dev.pool)
    gk, _ = dev.pools_host()
    keep = [0, 3]
    rk, _ = oracle.oracle_write(wl.write_k[keep], wl.write_v[keep], "f16", slots[keep],
                                wl.k_pool, wl.v_pool, "f16")
    assert np.array_equal(gk, rk)
    assert not np.array_equal(gk, before_k)


def test_copy_bitexact_and_cow_flow():
    wl = W.config4(num_blocks=2048)
    say(f"[copy] pairs={len(wl.copy_pairs)}")
    dev = DeviceWorkload(wl, tables=wl.tables_before_copy)
    before = out_f64(dev.decode())
    dev.copy()
    gk, gv = dev.pools_host()
    rk, rv = oracle.oracle_copy(wl.k_pool, wl.v_pool, wl.copy_pairs)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    dev.set_tables(wl.block_tables)
    after = out_f64(dev.decode())
    assert np.array_equal(before, after)          # the copies hold the same bytes
    ref = oracle_out(wl, k_pool=rk, v_pool=rv)
    assert max_err(after, ref) <= 2e-2
    # pairs outside the pool or with src == dst are skipped
    bad = torch.tensor([[0, wl.num_blocks], [-1, 3], [5, 5]], dtype=torch.int64, device=DEV)
    pa.pa_copy_blocks(dev.pool, bad)
    gk2, gv2 = dev.pools_host()
    assert np.array_equal(gk2, gk) and np.array_equal(gv2, gv)


# ---------------------------------------------------------------------------
# invariance, determinism, poison, edge cases
# ---------------------------------------------------------------------------

def test_relabelled_blocks_give_identical_bits():
    wl = W.config2(seed=21, num_seqs=6, ctx_range=(1, 600), num_blocks=512)
    other = W.relocate(wl, seed=22)
    a, b = DeviceWorkload(wl), DeviceWorkload(other)
    for p in (0, 16, 64, 512, pa.PA_PARTITION_AUTO):
        x = a.decode(partition_size=p).cpu()
        y = b.decode(partition_size=p).cpu()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), p


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_negative_and_zero_scale(scale):
    """Any finite scale, on the matrix-core path (single pass, balanced and
    fixed splits) and the generic one."""
    for kv, d in (("bf16", 128), ("bf16", 64)):
        wl = W.build_decode(70, name="scale", q_dtype="bf16", kv_dtype=kv, num_q_heads=32, num_kv_heads=8,
                            head_dim=d, block_size=16, num_blocks=600,
                            context_lens=np.array([1, 17, 300, 1500, 2000], np.int32),
                            rng=np.random.default_rng(70), poison=True)
        wl.scale = scale
        check_decode(wl, parts=(0, pa.PA_PARTITION_AUTO, 256), label=f"scale {scale} D={d}")


def test_deterministic_repeats():
    wl = W.config2(seed=23, num_seqs=5, ctx_range=(100, 900), num_blocks=512)
    dev = DeviceWorkload(wl)
    for p in (0, 128, pa.PA_PARTITION_AUTO):
        x = dev.decode(partition_size=p).cpu()
        for _ in range(3):
            assert torch.equal(x.view(torch.int16), dev.decode(partition_size=p).cpu().view(torch.int16))


@pytest.mark.parametrize("which", ["bf16", "f16", "fp8"])
def test_poisoned_unused_memory_is_never_used(which):
    if which == "fp8":
        rng = np.random.default_rng(31)
        lens = np.array([1, 31, 32, 33, 300])
        wl = W.build_write_filled(31, name="poison-fp8", q_dtype="bf16", src_dtype="bf16",
                                  kv_dtype="fp8_e4m3", num_q_heads=16, num_kv_heads=2, head_dim=128,
                                  block_size=32, num_blocks=40, context_lens=lens, rng=rng, poison=True)
    elif which == "bf16":
        wl = W.config2(seed=32, num_seqs=6, ctx_range=(1, 200), num_blocks=128, poison=True)
    else:
        wl = W.config3(seed=33, num_seqs=5, num_blocks=256, length_cap=120, poison=True)
        wl.write_k = wl.write_v = wl.slot_mapping = None        # decode only
    outs = check_decode(wl, parts=(0, wl.block_size, 512 if 512 % wl.block_size == 0 else 0,
                                   pa.PA_PARTITION_AUTO))
    for o in outs:
        assert np.isfinite(o).all()


def test_edge_lengths():
    bs, maxb = 16, 5
    lens = np.array([0, 1, bs, maxb * bs, 2, 0], dtype=np.int32)
    need = sum(-(-int(n) // bs) for n in lens)
    rng = np.random.default_rng(41)
    wl = W.build_decode(41, name="edges", q_dtype="bf16", kv_dtype="bf16", num_q_heads=8,
                        num_kv_heads=2, head_dim=128, block_size=bs, num_blocks=need + 2,
                        context_lens=lens, rng=rng, max_blocks_per_seq=maxb)
    outs = check_decode(wl, parts=(0, 16, 32, pa.PA_PARTITION_AUTO))
    for o in outs:
        assert not o[0].any() and not o[5].any()          # n == 0: zero rows


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_many_short_contexts(kv):
    """Over a thousand 1-2 tile contexts: in the balanced split a wave's tile
    range then spans about ten (sequence, head group) units, past the ones
    whose q is staged ahead, with whole units and split ones mixed.  With
    fixed partitions of one and two blocks, the split's workgroups find their
    items across 19 chunks of 64 sequences (chunks passed four at a time)."""
    rng = np.random.default_rng(51)
    lens = rng.integers(1, 25, size=1200)
    need = sum(-(-int(n) // 16) for n in lens)
    common = dict(q_dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                  num_blocks=need + 3, context_lens=lens, rng=rng)
    if kv == "bf16":
        wl = W.build_decode(51, name="short", kv_dtype="bf16", **common)
    else:
        wl = W.build_write_filled(51, name="short-fp8", src_dtype="bf16", kv_dtype="fp8_e4m3", **common)
    check_decode(wl, parts=(0, 16, 32, pa.PA_PARTITION_AUTO))


def test_out_of_range_table_entry_and_length_give_nan_rows():
    """Forced from the host: one sequence names a block past the pool, one
    has a length past its table.  The kernels' guards turn both into NaN rows
    (no out-of-bounds access); the other sequences stay exact."""
    wl = W.config2(seed=42, num_seqs=4, ctx_range=(20, 100), num_blocks=64)
    tables = wl.block_tables.copy()
    tables[1, 0] = wl.num_blocks + 7
    lens = wl.context_lens.copy()
    lens[2] = tables.shape[1] * wl.block_size + 1
    dev = DeviceWorkload(wl, tables=tables)
    dev.ctx = torch.from_numpy(lens).to(DEV)
    ref = oracle_out(wl)
    for p in (0, 32, pa.PA_PARTITION_AUTO):
        got = out_f64(dev.decode(partition_size=p))
        assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
        assert max_err(got[[0, 3]], ref[[0, 3]]) <= 2e-2


def test_nondefault_stream():
    wl = W.config2(seed=43, num_seqs=3, ctx_range=(10, 300), num_blocks=128)
    dev = DeviceWorkload(wl)
    ref = oracle_out(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, partition_size=64,
                           stream=s)
    s.synchronize()
    assert max_err(out_f64(out), ref) <= 2e-2


@pytest.mark.parametrize("part", [64, pa.PA_PARTITION_AUTO])
def test_stream_argument_not_current(part):
    """stream=s without making s current: the workspace the binding allocates
    is zero-filled on s itself, ahead of the kernels, and held until they end."""
    wl = W.config2(seed=45, num_seqs=5, ctx_range=(10, 700), num_blocks=256)
    dev = DeviceWorkload(wl)
    ref = oracle_out(wl)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        out = torch.full_like(dev.q, float("nan"))
        s.wait_stream(torch.cuda.current_stream())
        pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, out=out, partition_size=part,
                     q_dtype=wl.q_dtype, stream=s)
        s.synchronize()
        outs.append(out_f64(out))
    for got in outs:
        assert max_err(got, ref) <= 2e-2
        assert np.array_equal(got, outs[0])


# ---------------------------------------------------------------------------
# the balanced split's placement check, forced from the host through the
# workspace's control words (int32 index 32 * (1 + x): XCD x's registration
# count; 32 * 17: the poison word)
# ---------------------------------------------------------------------------

def _auto_ws(wl):
    return pa.new_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                            wl.max_blocks_per_seq, wl.block_size, pa.PA_PARTITION_AUTO, device=DEV)


def _auto(dev, ws):
    out = torch.full_like(dev.q, float("nan"))
    return out_f64(pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, dev.wl.scale, out=out,
                                partition_size=pa.PA_PARTITION_AUTO, workspace=ws,
                                q_dtype=dev.wl.q_dtype))


@pytest.mark.parametrize("surplus", ["one_xcd", "every_xcd", "poison_word"])
def test_placement_check_marks_workspace_until_zeroed(surplus):
    """A workgroup that draws an index past its XCD's share (as it would if
    the dispatcher did not deal workgroups to the XCDs in turn) writes NaN
    rows and marks the workspace; a marked workspace gives NaN rows until it
    is zero-filled, and then the results are exact again."""
    wl = W.config2(seed=44, num_seqs=6, ctx_range=(10, 500), num_blocks=256)
    dev = DeviceWorkload(wl)
    ref = oracle_out(wl)
    ws = _auto_ws(wl)
    assert max_err(_auto(dev, ws), ref) <= 2e-2
    assert pa.pa_decode_status(ws, pa.PA_PARTITION_AUTO) == pa.PA_WS_CLEAN
    words = ws.view(torch.int32)
    if surplus == "one_xcd":
        words[32 * 1] = 1 << 20
    elif surplus == "every_xcd":
        for x in range(16):
            words[32 * (1 + x)] = 1 << 20
    else:
        words[32 * 17] = 1
    got = _auto(dev, ws)
    if surplus == "one_xcd":
        assert np.isnan(got).any()
    else:
        assert np.isnan(got).all()
    assert int(words[32 * 17].item()) == 1
    assert pa.pa_decode_status(ws, pa.PA_PARTITION_AUTO) == pa.PA_WS_MISPLACED
    assert np.isnan(_auto(dev, ws)).all()           # marked: every row NaN
    ws.zero_()
    for _ in range(2):
        assert max_err(_auto(dev, ws), ref) <= 2e-2
    assert pa.pa_decode_status(ws, pa.PA_PARTITION_AUTO) == pa.PA_WS_CLEAN


def test_wait_bound_gives_up_marks_and_exits():
    """The balanced split's waits between the waves of a workgroup are
    bounded.  With the bound forced down to one poll from the host, waits
    that would normally last microseconds give up: the launch still ends
    (every wave exits), the status word says PA_WS_TIMED_OUT, rows are NaN
    rather than stale, later calls give NaN rows until the workspace is
    zero-filled, and then the results are exact again."""
    wl = W.config2(seed=46, num_seqs=8, ctx_range=(300, 1200), num_blocks=700)
    dev = DeviceWorkload(wl)
    ref = oracle_out(wl)
    ws = _auto_ws(wl)
    say("[wait bound] one poll")
    pa.pa_set_wait_polls(1)
    try:
        got = _auto(dev, ws)
    finally:
        pa.pa_set_wait_polls(0)
    torch.cuda.synchronize()
    assert pa.pa_decode_status(ws, pa.PA_PARTITION_AUTO) == pa.PA_WS_TIMED_OUT
    assert np.isnan(got).any()
    assert np.isnan(_auto(dev, ws)).all()           # marked: every row NaN
    ws.zero_()
    assert max_err(_auto(dev, ws), ref) <= 2e-2
    assert pa.pa_decode_status(ws, pa.PA_PARTITION_AUTO) == pa.PA_WS_CLEAN
    assert pa.pa_decode_status(ws, 64) == pa.PA_WS_CLEAN      # other modes keep no status


@pytest.mark.parametrize("part", [pa.PA_PARTITION_AUTO, 64])
def test_workspace_reused_across_batches(part):
    """One workspace, sized for the largest, through calls on different
    batches (different numbers of sequences, tiles and split units): each
    call finds its counters at zero although earlier calls used the same
    bytes differently, and each result matches the oracle and repeats bit for
    bit."""
    wls = [W.config2(seed=61, num_seqs=7, ctx_range=(1, 700), num_blocks=400),
           W.config2(seed=62, num_seqs=3, ctx_range=(300, 1200), num_blocks=300),
           W.config2(seed=63, num_seqs=12, ctx_range=(1, 90), num_blocks=100)]
    sizes = [pa.pa_decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                          w.max_blocks_per_seq, w.block_size, part)
             for w in wls]
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device=DEV)
    devs = [DeviceWorkload(w) for w in wls]
    refs = [oracle_out(w) for w in wls]
    first = [None] * len(wls)
    for rnd in range(3):
        for i, (w, dev) in enumerate(zip(wls, devs)):
            out = torch.full_like(dev.q, float("nan"))
            got = out_f64(pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, w.scale, out=out,
                                       partition_size=part, workspace=ws, q_dtype=w.q_dtype))
            assert max_err(got, refs[i]) <= 2e-2, (rnd, i)
            if first[i] is None:
                first[i] = got
            else:
                assert np.array_equal(got, first[i]), (rnd, i)
    if part == pa.PA_PARTITION_AUTO:
        assert int(ws.view(torch.int32)[32 * 17].item()) == 0  # never marked


@pytest.mark.parametrize("d", [128, 64])
def test_fixed_split_never_reads_stale_partials(d):
    """Fixed partitions with every byte of the workspace past its counters
    set to NaN beforehand (the counters zero, as the workspace contract asks):
    a call merges only the partials it has written itself, so the result
    matches the oracle and, bit for bit, the same call on clean scratch.
    d 128 runs the head-dim-128 split and its merge launch, d 64 the generic
    kernels."""
    rng = np.random.default_rng(71 + d)
    bs = 16
    lens = np.concatenate([[1, bs, bs + 1, 200], rng.integers(1, 400, size=5)])
    need = sum(-(-int(n) // bs) for n in lens)
    wl = W.build_decode(71 + d, name=f"stale-{d}", q_dtype="bf16", kv_dtype="bf16", num_q_heads=8,
                        num_kv_heads=2, head_dim=d, block_size=bs, num_blocks=need + 5,
                        context_lens=lens, rng=rng)
    dev = DeviceWorkload(wl)
    ref = oracle_out(wl)
    units = wl.num_seqs * wl.num_kv_heads          # group 4: one head group per KV head
    counter_bytes = -(-(units * 8) // 256) * 256
    for part in (bs, 64):
        size = pa.pa_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, d,
                                            wl.max_blocks_per_seq, bs, part)
        say(f"[stale partials] d={d} partition {part} workspace {size} B")
        clean = torch.zeros(size, dtype=torch.uint8, device=DEV)
        stale = torch.full((size,), 0xFF, dtype=torch.uint8, device=DEV)
        stale[:counter_bytes] = 0
        outs = []
        for ws in (clean, stale):
            out = torch.full_like(dev.q, float("nan"))
            got = out_f64(pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, out=out,
                                       partition_size=part, workspace=ws, q_dtype=wl.q_dtype))
            assert np.isfinite(got).all(), part
            assert max_err(got, ref) <= 2e-2, part
            outs.append(got)
        assert np.array_equal(outs[0], outs[1]), part


@pytest.mark.parametrize("part", [pa.PA_PARTITION_AUTO, 0, 64])
def test_timed_decode_records_its_kernels(part):
    """pa_time_next_decode: the event pair brackets the call's kernels (a
    positive time no longer than a bracket around the whole call) and the
    result is unchanged."""
    wl = W.config2(seed=71, num_seqs=5, ctx_range=(50, 900), num_blocks=300)
    dev = DeviceWorkload(wl)
    ref = oracle_out(wl)
    st = torch.cuda.current_stream()
    k0, k1, b0, b1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    for e in (k0, k1):
        e.record(st)                   # creates the events
    torch.cuda.synchronize()
    ws = pa.new_workspace(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.max_blocks_per_seq,
                          wl.block_size, part, device=DEV) if part else None
    out = torch.full_like(dev.q, float("nan"))
    b0.record(st)
    pa.pa_time_next_decode(k0, k1)
    pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, out=out, partition_size=part,
                 workspace=ws, q_dtype=wl.q_dtype, stream=st)
    b1.record(st)
    torch.cuda.synchronize()
    kernel_ms, bracket_ms = k0.elapsed_time(k1), b0.elapsed_time(b1)
    say(f"    partition {part}: kernels {kernel_ms * 1e3:.1f} us, bracket {bracket_ms * 1e3:.1f} us")
    assert 0 < kernel_ms <= bracket_ms
    assert max_err(out_f64(out), ref) <= 2e-2
    # the same with the timing-only events bench.py hands to the hook
    import bench
    t0, t1 = bench.TimingEvent(), bench.TimingEvent()
    out.fill_(float("nan"))
    b0.record(st)
    pa.pa_time_next_decode(t0, t1)
    pa.pa_decode(dev.q, dev.pool, dev.tables, dev.ctx, wl.scale, out=out, partition_size=part,
                 workspace=ws, q_dtype=wl.q_dtype, stream=st)
    b1.record(st)
    torch.cuda.synchronize()
    timing_ms, bracket_ms = t0.elapsed_time(t1), b0.elapsed_time(b1)
    say(f"    partition {part}: kernels (timing-only events) {timing_ms * 1e3:.1f} us")
    assert 0 < timing_ms <= bracket_ms
    assert max_err(out_f64(out), ref) <= 2e-2
