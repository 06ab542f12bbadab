"""Each planted mistake in a copy of the oracle must fail at least one pin.

The mistakes are the plausible ones: a wrong GQA head mapping, a dropped
scale, no truncation to context_len, a transposed gather, a flipped softmax
sign, wrong fp8 constants or tie rule (saturation has no
single-line mistake: the index clip saturates even without the clamp), a swapped per-tensor scale, a wrong
slot decomposition, a flipped merge weight, a dropped merge normaliser.  The
copies are made from the oracle's source text on the CPU; the oracle itself
is untouched.
"""

import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "pa_oracle.py")

MUTANTS = [
    ("gqa-mapping", "kvh = h // group", "kvh = h % num_kv_heads"),
    ("dropped-scale", "z = scale64 * (k[kvh] @ qf[s, h])", "z = (k[kvh] @ qf[s, h])"),
    ("no-truncation", "return per_head[:, :num_tokens, :]", "return per_head"),
    ("transposed-gather", "blocks.transpose(1, 0, 2, 3)", "blocks.transpose(0, 1, 2, 3)"),
    ("softmax-sign", "p = np.exp(z - z.max())", "p = np.exp(z.max() - z)"),
    ("missing-normaliser", "out[s, h] = (p @ v[kvh]) / p.sum()", "out[s, h] = (p @ v[kvh])"),
    ("e4m3-subnormal", "(mantissa / 8.0) * 2.0 ** (1 - 7)", "(mantissa / 8.0) * 2.0 ** (0 - 7)"),
    ("e4m3-bias", "2.0 ** (exponent - 7)", "2.0 ** (exponent - 8)"),
    ("e4m3-ties", "(hi % 2 == 0)", "(hi % 2 == 1)"),
    ("scale-swap", "v = v * float(np.float32(v_scale))", "v = v * float(np.float32(k_scale))"),
    ("inverse-scale", "inv = np.float32(1.0) / np.float32(sc)", "inv = np.float32(sc)"),
    ("slot-split", "blk, off = slots // block_size, slots % block_size",
     "blk, off = slots % block_size, slots // block_size"),
    ("merge-weight", "w = np.exp(m[s, h, :P] - big_m)", "w = np.exp(big_m - m[s, h, :P])"),
    ("merge-denominator", "(w @ o[s, h, :P]) / (w @ l[s, h, :P])", "(w @ o[s, h, :P]) / l[s, h, :P].sum()"),
    ("partition-bound", "lo, hi = p * partition_size, min((p + 1) * partition_size, n)",
     "lo, hi = p * partition_size, min((p + 1) * partition_size + 1, n)"),
    ("bf16-shift", "<< np.uint32(16)\n        return bits.view(np.float32).astype(np.float64)",
     "<< np.uint32(15)\n        return bits.view(np.float32).astype(np.float64)"),
    ("copy-direction", "k_pool[dst] = k_pool[src]", "k_pool[src] = k_pool[dst]"),
    ("blocks-floor", "return -(-num_tokens // block_size)", "return num_tokens // block_size"),
    ("window-bound", "return max(0, n - window) if window else 0",
     "return max(0, n - window - 1) if window else 0"),
    ("range-offset", "off = start - first * block_size", "off = start - first"),
    ("causal-limit", "z = scale64 * (k[kvh, lo - first:p + 1 - first]",
     "z = scale64 * (k[kvh, lo - first:p + 2 - first]"),
    ("query-position", "p = n - L + i", "p = i"),
    ("prefill-group", "kvh = h // group\n                z = scale64 * (k[kvh, lo",
     "kvh = h % num_kv_heads\n                z = scale64 * (k[kvh, lo"),
    ("swap-direction", "dst_k[dst] = src_k[src]", "dst_k[dst] = dst_k[src]"),
    ("decode-scale-magnitude", "    scale64 = float(np.float32(scale))\n    qf = to_float64(q, q_dtype)\n    out = np.zeros((num_seqs,",
     "    scale64 = abs(float(np.float32(scale)))\n    qf = to_float64(q, q_dtype)\n    out = np.zeros((num_seqs,"),
    ("prefill-scale-magnitude", "    scale64 = float(np.float32(scale))\n    qf = to_float64(q, q_dtype)\n    out = np.zeros((num_tokens,",
     "    scale64 = abs(float(np.float32(scale)))\n    qf = to_float64(q, q_dtype)\n    out = np.zeros((num_tokens,"),
]


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"pattern not found: {old!r}"
    mod = types.ModuleType("pa_oracle_mutant")
    exec(compile(src.replace(old, new), SRC + ":mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutant(old, new)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:                      # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
