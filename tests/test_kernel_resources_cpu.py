"""The attention kernels keep the occupancy their designs are built on.

Each bf16 attention kernel is designed for a number of waves per SIMD: two
4-wave prefill workgroups per CU, or one 8-wave workgroup with two key-tile
groups; two decode waves per SIMD, each with two tiles of loads in flight;
the fused mixed-batch kernel like the prefill kernel.  A change that adds
registers or LDS can halve that silently (results stay right, the rate
drops), so this test compiles the sources to gfx950 assembly with the
library's flags and reads, per kernel, the compiler's occupancy (waves per
SIMD allowed by the registers), the LDS a workgroup takes (160 KB per CU on
this part) and the scratch bytes per lane.  CPU only (hipcc cross-compiles).
"""

import os
import re
import shutil
import subprocess

import pytest

from decode_paged_kv_amd import build

CSRC = os.path.join(os.path.dirname(build.__file__), "csrc")
LDS_PER_CU = 160 * 1024
SIMDS_PER_CU = 4

# (source, kernel name pattern, waves per workgroup, waves per SIMD at
# least, scratch allowed).  The prefill kernels spill a few registers on
# their ragged-tail and epilogue paths, outside the tile loop.
CASES = [
    ("attn_prefill.hip", "attn_prefill_bf16_kernelILi128ELi1E", 4, 2, True),
    ("attn_prefill.hip", "attn_prefill_bf16_kernelILi64ELi1E", 4, 2, True),
    ("attn_prefill.hip", "attn_prefill_bf16_kernelILi128ELi2E", 8, 2, True),
    ("attn_prefill.hip", "attn_prefill_bf16_kernelILi64ELi2E", 8, 2, True),
    ("attn_decode.hip", "attn_decode_bf16_kernel", 4, 2, False),
    ("attn_decode.hip", "attn_decode_line_kernel", 4, 2, False),
    ("attn_mixed.hip", "attn_mixed_bf16_kernel", 4, 2, False),
]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("res")
    flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"]
    procs = {}
    for src in sorted({c[0] for c in CASES}):
        out = str(d / (src + ".s"))
        procs[src] = (out, subprocess.Popen([hipcc, "-x", "hip", *flags, "--offload-device-only", "-S",
                                             os.path.join(CSRC, src), "-o", out],
                                            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    texts = {}
    for src, (out, p) in procs.items():
        _, err = p.communicate()
        assert p.returncode == 0, err[-4000:]
        with open(out) as f:
            texts[src] = f.read()
    return texts


def resources(text, pattern):
    """(name, waves per SIMD the registers allow, LDS bytes, scratch bytes) per matching kernel."""
    labels = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w+):", text, re.M)]
    out = []
    for i, (at, name) in enumerate(labels):
        if pattern not in name:
            continue
        end = labels[i + 1][0] if i + 1 < len(labels) else len(text)
        part = text[at:end]
        occ = int(re.search(r"; Occupancy: (\d+)", part).group(1))
        lds = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", part).group(1))
        scratch = int(re.search(r"; ScratchSize: (\d+)", part).group(1))
        out.append((name, occ, lds, scratch))
    return out


def waves_per_simd(occ, lds, wg_waves):
    """Waves per SIMD a kernel can hold: the lower of the register bound and the LDS bound."""
    by_lds = (LDS_PER_CU // lds) * wg_waves // SIMDS_PER_CU if lds else occ
    return min(occ, by_lds)


@pytest.mark.parametrize("src,pattern,wg_waves,min_waves,scratch_ok", CASES)
def test_kernel_keeps_its_occupancy(asm, src, pattern, wg_waves, min_waves, scratch_ok):
    found = resources(asm[src], pattern)
    assert found, pattern
    for name, occ, lds, scratch in found:
        w = waves_per_simd(occ, lds, wg_waves)
        assert w >= min_waves, f"{name}: {w} waves per SIMD (registers allow {occ}, LDS {lds} B)"
        if not scratch_ok:
            assert scratch == 0, f"{name}: {scratch} scratch bytes per lane"


def test_lds_bound_is_applied():
    # a 4-wave workgroup of 82 KB fits once per CU: one wave per SIMD, even
    # where the registers would allow two (the mixed-batch kernel's LDS at
    # G = 8 when its two bodies' LDS was summed)
    assert waves_per_simd(2, 82208, 4) == 1
    assert waves_per_simd(2, 65536, 4) == 2
    assert waves_per_simd(2, 131072, 8) == 2
    assert waves_per_simd(1, 0, 4) == 1
