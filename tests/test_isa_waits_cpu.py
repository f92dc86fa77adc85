"""The whole-line K decode kernels wait for their loads before any use.

Their K/V/q loads and LDS reads are inline assembly with explicit wait
counts (the compiler's own waits would keep one tile in flight per wave
instead of two).  The kernels are compiled to gfx950 assembly with the
library's flags and checked by tests/isa_waits.py: on no path does an
instruction other than a wait name a register that a load in flight has yet
to fill, and nothing is spilled to scratch.  The checker itself is checked
on a planted early use.  CPU only (hipcc cross-compiles).
"""

import os
import re
import shutil
import subprocess

import pytest

import isa_waits
from decode_paged_kv_amd import build

SRC = os.path.join(os.path.dirname(build.__file__), "csrc", "attn_decode.hip")

PLANTED = """k:
\tbuffer_load_dwordx4 v[0:3], v10, s[0:3], s4 offen nt
\tbuffer_load_dwordx2 v[4:5], v10, s[0:3], s4 offen nt
\ts_waitcnt vmcnt(1)
\tv_mov_b32 v6, v0
\tv_mov_b32 v7, v4
.LBB0_1:
\tbuffer_load_dwordx4 v[20:23], v10, s[0:3], s4 offen nt
\tds_read_b128 v[30:33], v11
\ts_waitcnt vmcnt(1) lgkmcnt(0)
\tv_add_f32_e32 v8, v20, v30
\ts_cbranch_scc1 .LBB0_1
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
"""


def test_checker_finds_planted_early_uses():
    issues = isa_waits.check(PLANTED, "k")
    # v4 read while its load is in flight; v20 read with the loop's own load
    # still in flight (the wait leaves one); v0 and v30 are valid
    assert sorted({tuple(i[2]) for i in issues}) == [(4,), (20,)]


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "attn_decode.s")
    flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"]
    res = subprocess.run([hipcc, "-x", "hip", *flags, "--offload-device-only", "-S", SRC, "-o", out],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    with open(out) as f:
        return f.read()


def test_line_kernels_wait_before_every_use(decode_asm):
    names = isa_waits.kernels(decode_asm, "attn_decode_line_kernel")
    assert len(names) == 20                       # head dims {64, 128} x groups {1..16} x append
    for n in names:
        issues = isa_waits.check(decode_asm, n)
        assert not issues, f"{n}: {issues[:5]}"


def test_line_kernels_do_not_spill(decode_asm):
    for n in isa_waits.kernels(decode_asm, "attn_decode_line_kernel"):
        at = decode_asm.index(n + ":")
        m = re.search(r"; ScratchSize: (\d+)", decode_asm[at:])
        assert m and int(m.group(1)) == 0, n
