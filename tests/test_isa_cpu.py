"""Code-generation guards for the head-dim-128 kernels (CPU only): the
balanced-split decode kernel's schedule, and the prefill kernels' registers.

The streaming wave keeps two K/V tiles (16 loads) in flight while it computes
the current one.  That depends on the tile loop's cursor staying in scalar
registers: once the compiler treats it as per-lane, table entries and
context lengths become vector loads, and each such load waits for every
tile load issued before it, which cost a third of the kernel's speed once.
The first tests compile the decode kernels to gfx950 assembly and check
the signature of the intended schedule in decode_pair_kernel<bf16, bf16,
group 4, block 16>, the kernel the Llama-3-8B-shaped layer runs:

* the first waits inside the tile loop leave 14 loads outstanding;
* no vector dword load inside the tile loop (the lengths and table entries
  it reads are scalar loads), and only a few in the whole kernel (set-up and
  merge).
"""

import os
import re
import subprocess

import pytest

from paged_kv_cache_91_amd import build as B

KERNEL = "_ZN7pa_impl12_GLOBAL__N_118decode_pair_kernelINS0_5BF16SES2_Li4ELi16ELb0EEEvPKiPiiiiiiNS_10DecodeArgsE"


@pytest.fixture(scope="module")
def pair_isa(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "k.s"
    cmd = [B.hipcc(), *B.FLAGS, "-DPA_FAST_COMBO=0", "--cuda-device-only", "-S",
           os.path.join(B.PKG, "csrc", "pa_decode_fast.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("hipcc unavailable: " + res.stderr[-300:])
    text = out.read_text()
    start = text.index(KERNEL + ":")
    end = text.index(".Lfunc_end", start)
    return text[start:end]


def test_tile_loop_keeps_two_tiles_in_flight(pair_isa):
    lines = pair_isa.splitlines()
    first_mfma = next(i for i, l in enumerate(lines) if "v_mfma_f32_16x16x32" in l)
    waits = [int(m.group(1)) for l in lines[first_mfma:first_mfma + 200]
             for m in [re.search(r"s_waitcnt vmcnt\((\d+)\)", l)] if m]
    assert waits and max(waits[:3]) >= 12, waits[:8]


def _loops_with_mfma(lines):
    """(first, last) line of every loop (a backward branch) whose body holds an MFMA."""
    labels = {m.group(1): i for i, l in enumerate(lines) for m in [re.match(r"^(\.LBB\w+):", l)] if m}
    loops = []
    for i, l in enumerate(lines):
        m = re.search(r"s_c?branch\w*\s+(\.LBB\w+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            body = lines[labels[m.group(1)]:i + 1]
            if any("v_mfma" in b for b in body):
                loops.append((labels[m.group(1)], i))
    return loops


def test_tile_loop_reads_tables_and_lengths_with_scalar_loads(pair_isa):
    lines = pair_isa.splitlines()
    loops = _loops_with_mfma(lines)
    assert loops
    first, last = min(a for a, _ in loops), max(b for _, b in loops)
    in_loop = [l for l in lines[first:last + 1] if re.search(r"\bglobal_load_dword\s", l)]
    assert not in_loop, in_loop
    vector_dword_loads = len(re.findall(r"\bglobal_load_dword\s", pair_isa))
    assert vector_dword_loads <= 16, vector_dword_loads


# Prefill: the prefetched K/V chunks once went through scratch memory (an
# array in a lambda), which also made every tile wait for its loads at once,
# and register growth past 168 drops the kernel from three waves per SIMD to
# two (both measured several percent).  Every prefill specialisation must
# compile with no scratch and at most 168 VGPRs.
PREFILL_MAX_VGPRS = 168


@pytest.fixture(scope="module")
def prefill_resources(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "pf.o"
    cmd = [B.hipcc(), *B.FLAGS, "--cuda-device-only", "-c", os.path.join(B.PKG, "csrc", "pa_prefill.hip"),
           "-o", str(out), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("hipcc unavailable: " + res.stderr[-300:])
    kernels = {}
    for block in res.stderr.split("Function Name: ")[1:]:
        name = block.split()[0]
        vgpr = int(re.search(r"VGPRs: (\d+)", block).group(1))
        scratch = int(re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block).group(1))
        kernels[name] = (vgpr, scratch)
    return kernels


def test_prefill_kernels_keep_three_waves_per_simd_without_scratch(prefill_resources):
    pf = {k: v for k, v in prefill_resources.items() if "prefill_kernel" in k}
    assert len(pf) == 16, sorted(pf)                    # bf16/f16 x block 16/32 x group 1/2/4/8
    for name, (vgpr, scratch) in pf.items():
        assert scratch == 0, (name, scratch)
        assert vgpr <= PREFILL_MAX_VGPRS, (name, vgpr)


@pytest.fixture(scope="module", params=[0, 2], ids=["bf16-bf16", "bf16-fp8"])
def decode_resources(request, tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "df.o"
    cmd = [B.hipcc(), *B.FLAGS, f"-DPA_FAST_COMBO={request.param}", "--cuda-device-only", "-c",
           os.path.join(B.PKG, "csrc", "pa_decode_fast.hip"), "-o", str(out),
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("hipcc unavailable: " + res.stderr[-300:])
    kernels = {}
    for block in res.stderr.split("Function Name: ")[1:]:
        name = block.split()[0]
        scratch = int(re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block).group(1))
        kernels[name] = scratch
    return kernels


def test_decode_kernels_use_no_scratch(decode_resources):
    """Every head-dim-128 decode kernel (the balanced split, the single pass,
    the fixed split at its three waves per SIMD, the merge) fits its
    registers: a spill to scratch memory in the fixed split's item search
    once made that kernel a quarter slower."""
    kinds = ("decode_pair_kernel", "decode_fast_kernel", "decode_split_kernel", "merge_parts_kernel")
    found = {k: 0 for k in kinds}
    for name, scratch in decode_resources.items():
        for k in kinds:
            if k in name:
                found[k] += 1
                assert scratch == 0, (name, scratch)
    assert all(found.values()), found
