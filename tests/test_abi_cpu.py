"""Boundary checks that need no GPU.

* libpkv.so loads and exports every function include/pkv.h declares;
* the binding's signature table covers exactly those functions;
* invalid arguments are rejected on the host with the documented codes,
  before any HIP call (nothing here touches a device).
"""

import ctypes as C
import os
import re
import subprocess

import pytest

from conftest import ROOT

lib_mod = pytest.importorskip("decode_paged_kv_amd._lib")


def _lib():
    if not os.path.exists(lib_mod.LIB_PATH):
        pytest.skip("libpkv.so not built (run python -m decode_paged_kv_amd.build)")
    return lib_mod.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"typedef struct \w+ \{.*?\} \w+;", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_every_declared_symbol_is_exported():
    _lib()
    declared = _declared_functions()
    # the calls the boundary is built around, and nothing declared twice
    required = {"kv_write", "kv_relayout", "attn_prefill_chunk", "attn_decode", "pkv_attn_decode_workspace_size",
                "run_mux_round", "pkv_mux_create", "pkv_mux_groups", "pkv_mux_choose", "pkv_mux_layers_per_round",
                "pkv_mux_stream", "pkv_mux_destroy", "pkv_last_error"}
    assert required <= set(declared), required - set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", lib_mod.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in declared if n not in exported]
    assert not missing, missing
    assert sorted(lib_mod.EXPORTED) == declared


def test_calibration_library_exports_and_rejects_bad_arguments():
    """The benchmark's calibration kernels (libpkv_calib.so): exported, and argument errors come back from the
    host side as hipErrorInvalidValue (1) before any launch."""
    from decode_paged_kv_amd import build as b
    if not os.path.exists(b.CALIB_LIB):
        pytest.skip("libpkv_calib.so not built")
    out = subprocess.run(["nm", "-D", "--defined-only", b.CALIB_LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {"pkv_calib_mfma", "pkv_calib_mfma_random", "pkv_calib_tiled_read", "pkv_calib_tiled_copy",
            "pkv_calib_copy"} <= exported
    cl = C.CDLL(b.CALIB_LIB)
    cl.pkv_calib_tiled_read.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    cl.pkv_calib_tiled_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                        C.c_void_p]
    cl.pkv_calib_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
    cl.pkv_calib_mfma.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    cl.pkv_calib_mfma_random.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    fake = 0x100000
    assert cl.pkv_calib_tiled_read(None, fake, 1, 1, 8, fake, None) == 1
    assert cl.pkv_calib_tiled_read(fake, fake, 1, 1, 5, fake, None) == 1       # unroll not built
    assert cl.pkv_calib_tiled_copy(fake, fake, fake, fake, 1, 0, 4, None) == 1
    assert cl.pkv_calib_tiled_copy(fake, fake, fake, fake, 1, 1, 3, None) == 1
    assert cl.pkv_calib_copy(fake, fake, 24, 1, None) == 1                      # not a multiple of 16
    assert cl.pkv_calib_copy(fake + 8, fake, 32, 1, None) == 1                  # misaligned
    assert cl.pkv_calib_mfma(0, 1, fake, fake, None) == 1
    assert cl.pkv_calib_mfma_random(12, 1, fake, fake, None) == 1              # not a multiple of 8


def _pool(**kw):
    p = lib_mod.PoolLayer()
    p.num_blocks, p.block_size, p.num_kv_heads, p.num_shards, p.head_dim = 8, 16, 8, 4, 128
    p.dtype = lib_mod.BF16
    for s in range(4):
        p.k[s] = 0x10000 * (s + 1)
        p.v[s] = 0x10000 * (s + 10)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _err(lib):
    return lib.pkv_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("block_size", 24, -2), ("block_size", 8, -2), ("head_dim", 96, -2), ("num_shards", 3, -2),
    ("num_shards", 0, -1), ("num_shards", 17, -1), ("num_blocks", 0, -1), ("dtype", 7, -2), ("num_kv_heads", 0, -1),
])
def test_kv_write_rejects_bad_pool(field, value, code):
    lib = _lib()
    p = _pool(**{field: value})
    rc = lib.kv_write(C.byref(p), 0x1000, 0x2000, 0x3000, 4, None)
    assert rc == code, _err(lib)
    assert _err(lib)


def test_null_and_misaligned_pointers():
    lib = _lib()
    assert lib.kv_write(None, 0x1000, 0x2000, 0x3000, 4, None) == -1
    p = _pool()
    p.k[2] = 0
    assert lib.kv_write(C.byref(p), 0x1000, 0x2000, 0x3000, 4, None) == -1
    p = _pool()
    p.v[1] = 0x10008
    assert lib.kv_write(C.byref(p), 0x1000, 0x2000, 0x3000, 4, None) == -1
    assert lib.kv_write(C.byref(_pool()), 0x1004, 0x2000, 0x3000, 4, None) == -1
    assert lib.kv_write(C.byref(_pool()), 0, 0x2000, 0x3000, 4, None) == -1
    assert lib.kv_write(C.byref(_pool()), 0x1000, 0x2000, 0x3000, -1, None) == -1
    # zero tokens is a valid no-op
    assert lib.kv_write(C.byref(_pool()), 0, 0, 0, 0, None) == 0


def test_relayout_validation():
    lib = _lib()
    src = _pool()
    dst = _pool(block_size=32, num_shards=8)
    for s in range(8):
        dst.k[s] = 0x100000 * (s + 1)
        dst.v[s] = 0x100000 * (s + 20)
    bad = _pool(head_dim=64)
    assert lib.kv_relayout(C.byref(src), 0x10, C.byref(bad), 0x20, 16, None) == -1
    other = _pool(dtype=lib_mod.F32)
    assert lib.kv_relayout(C.byref(src), 0x10, C.byref(other), 0x20, 16, None) == -2
    assert lib.kv_relayout(C.byref(src), 0, C.byref(dst), 0x20, 16, None) == -1
    assert lib.kv_relayout(C.byref(src), 0x10, C.byref(dst), 0x20, 8 * 16 + 1, None) == -1   # does not fit
    same = _pool(block_size=32)
    assert lib.kv_relayout(C.byref(src), 0x10, C.byref(same), 0x20, 16, None) == -1           # shared buffers
    assert lib.kv_relayout(C.byref(src), 0x10, C.byref(dst), 0x20, 0, None) == 0


def _dest(**kw):
    d = lib_mod.KvDest()
    d.num_blocks, d.block_size, d.num_kv_heads, d.num_shards, d.head_dim = 8, 32, 8, 8, 128
    d.dtype, d.layout, d.scale = lib_mod.FP8_E4M3, lib_mod.LAYOUT_TOKEN_MAJOR, 0.25
    for s in range(8):
        d.k[s] = 0x100000 * (s + 1)
        d.v[s] = 0x100000 * (s + 20)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_relayout_convert_validation():
    lib = _lib()
    src = _pool()
    ok = lambda d, n=16, sbt=0x10: lib.kv_relayout_convert(C.byref(src), sbt, C.byref(d), 0x20, n, None)  # noqa
    assert ok(_dest(), 0) == 0                                   # zero tokens: a no-op
    assert lib.kv_relayout_convert(C.byref(src), 0x10, None, 0x20, 16, None) == -1
    assert ok(_dest(head_dim=64)) == -1
    assert ok(_dest(num_kv_heads=4)) == -1
    assert ok(_dest(block_size=8)) == -2 and ok(_dest(block_size=48)) == -2 and ok(_dest(block_size=256)) == -2
    assert ok(_dest(num_shards=3)) == -2 and ok(_dest(num_shards=0)) == -2
    assert ok(_dest(layout=3)) == -1
    assert ok(_dest(dtype=lib_mod.F32)) == -2                    # bf16 -> f32 is not a supported conversion
    assert ok(_dest(scale=0.0)) == -1 and ok(_dest(scale=float("inf"))) == -1 and ok(_dest(scale=float("nan"))) == -1
    assert ok(_dest(num_blocks=0)) == -1
    assert ok(_dest(), -1) == -1
    assert ok(_dest(), 16, 0) == -1                              # NULL source table
    assert ok(_dest(), 8 * 32 + 1) == -1                         # does not fit
    d = _dest()
    d.v[3] = 0
    assert ok(d) == -1                                           # NULL V buffer ...
    d.layout = lib_mod.LAYOUT_KV_FUSED
    assert ok(d, 0) == 0                                         # ... is fine when K and V are fused
    d = _dest()
    d.k[2] = 0x100008
    assert ok(d) == -1                                           # misaligned
    d = _dest()
    d.k[5] = src.v[1]
    assert ok(d) == -1                                           # shares a source buffer
    fp32src = _pool(dtype=lib_mod.F32)
    assert lib.kv_relayout_convert(C.byref(fp32src), 0x10, C.byref(_dest()), 0x20, 16, None) == -2   # fp8 from f32


def test_attention_validation():
    lib = _lib()
    p = _pool()
    # q-heads not a multiple of kv heads, or an unsupported group
    assert lib.attn_decode(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 2, 64, 12, 0.0, 0x500, 1 << 20, None) == -1
    assert lib.attn_decode(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 2, 64, 8 * 32, 0.0, 0x500, 1 << 20, None) == -2
    # table too narrow for the context
    assert lib.attn_decode(C.byref(p), 0x100, 0x200, 0x300, 2, 0x400, 2, 64, 32, 0.0, 0x500, 1 << 20, None) == -1
    # workspace too small when splits are needed
    need = lib.pkv_attn_decode_workspace_size(4, 32, 8192, 128)
    assert need > 0
    assert lib.attn_decode(C.byref(p), 0x100, 0x200, 0x300, 512, 0x400, 4, 8192, 32, 0.0, 0x500, 16, None) == -1
    assert lib.attn_decode(C.byref(p), 0x100, 0x200, 0x300, 512, 0x400, 4, 8192, 32, float("inf"), 0x500,
                           need, None) == -1
    assert lib.attn_decode(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 0, 64, 32, 0.0, 0, 0, None) == 0
    # append: the new rows must be there and aligned; otherwise as attn_decode
    ap = lambda kn, vn, bt_stride=8, scale=0.0: lib.attn_decode_append(  # noqa: E731
        C.byref(p), 0x100, kn, vn, 0x200, 0x300, bt_stride, 0x400, 2, 64, 32, scale, 0x500, 1 << 20, None)
    assert ap(0, 0x700) == -1 and ap(0x600, 0) == -1 and ap(0x608, 0x700) == -1
    assert ap(0x600, 0x700, bt_stride=2) == -1 and ap(0x600, 0x700, scale=float("nan")) == -1
    assert lib.attn_decode_append(C.byref(p), 0x100, 0x600, 0x700, 0x200, 0x300, 8, 0x400, 0, 64, 32, 0.0, 0, 0,
                                  None) == 0
    # a NaN or negative scale is rejected on the host (tested on the bits)
    for bad_scale in (float("nan"), -float("nan"), -0.5, float("-inf")):
        assert lib.attn_decode(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 2, 64, 32, bad_scale, 0x500, 1 << 20,
                               None) == -1
        assert lib.attn_prefill_chunk(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 0x500, 1, 64, 128, 32, bad_scale,
                                      None) == -1
    assert lib.attn_prefill_chunk(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 0x500, 1, 64, 128, 30, 0.0, None) == -1
    assert lib.attn_prefill_chunk(C.byref(p), 0x108, 0x200, 0x300, 8, 0x400, 0x500, 1, 64, 128, 32, 0.0, None) == -1
    assert lib.attn_prefill_chunk(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 0x500, 0, 64, 128, 32, 0.0, None) == 0
    # max_total_len: at least the chunk, and within what the table addresses (8 blocks x 16 = 128 keys)
    assert lib.attn_prefill_chunk(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 0x500, 1, 64, 63, 32, 0.0, None) == -1
    assert lib.attn_prefill_chunk(C.byref(p), 0x100, 0x200, 0x300, 8, 0x400, 0x500, 1, 64, 129, 32, 0.0, None) == -1
    assert "cannot hold" in _err(lib)
    # mixed batch: both parts empty is a no-op; each part is validated like its own entry point
    assert lib.attn_mixed_batch(C.byref(p), None, None, None, 0, None, 0, 0, None, None, None, 0, None, None, 0, 0,
                                0, 32, 0.0, None, 0, None) == 0
    assert lib.attn_mixed_batch(C.byref(p), 0x100, 0x200, None, 8, 0x400, 2, 64, None, None, None, 0, None, None,
                                0, 0, 0, 32, 0.0, 0x500, 1 << 20, None) == -1       # NULL decode table
    assert lib.attn_mixed_batch(C.byref(p), 0x100, 0x200, 0x300, 2, 0x400, 2, 64, None, None, None, 0, None, None,
                                0, 0, 0, 32, 0.0, 0x500, 1 << 20, None) == -1       # table too narrow
    assert lib.attn_mixed_batch(C.byref(p), None, None, None, 0, None, 0, 0, 0x108, 0x200, 0x300, 8, 0x400,
                                0x500, 1, 64, 128, 32, 0.0, None, 0, None) == -1    # misaligned prefill q
    assert lib.attn_mixed_batch(C.byref(p), None, None, None, 0, None, 0, 0, 0x100, 0x200, 0x300, 8, 0x400,
                                0x500, 1, 64, 128, 30, 0.0, None, 0, None) == -1    # heads not a multiple
    assert lib.attn_mixed_batch(C.byref(p), None, None, None, 0, None, 0, 0, 0x100, 0x200, 0x300, 8, 0x400,
                                0x500, 1, 64, 129, 32, 0.0, None, 0, None) == -1    # table below max_total_len
    assert lib.attn_mixed_batch(C.byref(p), 0x100, 0x200, 0x300, 512, 0x400, 4, 8192, None, None, None, 0, None,
                                None, 0, 0, 0, 32, 0.0, 0x500, 16, None) == -1      # workspace too small


def test_slot_mapping_validation():
    lib = _lib()
    assert lib.pkv_slot_mapping(0x10, 4, 0x20, 0x30, 0, 5, 16, 64, 0x40, None, None) == -1
    assert lib.pkv_slot_mapping(0x10, 4, 0x20, 0x30, 1, 5, 24, 64, 0x40, None, None) == -2
    assert lib.pkv_slot_mapping(0x10, 0, 0x20, 0x30, 1, 5, 16, 64, 0x40, None, None) == -1
    assert lib.pkv_slot_mapping(0, 0, 0, 0, 0, 0, 16, 64, 0, None, None) == 0


def test_workspace_size_is_zero_for_single_split():
    lib = _lib()
    assert lib.pkv_attn_decode_workspace_size(4, 4, 64, 64) == 0
    assert lib.pkv_attn_decode_workspace_size(0, 4, 128, 64) == 0


def test_workspace_size_for_a_pool_is_exact_and_within_the_worst_case():
    # the pool-aware query returns the plan of this pool's KV heads and dtype; the four-argument query is the
    # largest over every group size and both dtypes, so it is never smaller
    lib = _lib()
    for hkv, dtype in ((8, lib_mod.BF16), (8, lib_mod.F32), (2, lib_mod.BF16), (32, lib_mod.BF16)):
        p = _pool(num_kv_heads=hkv, num_shards=1, dtype=dtype)
        for batch, ctx in ((4, 8192), (16, 5000), (64, 512), (1, 100)):
            exact = lib.pkv_attn_decode_workspace_size_for(C.byref(p), batch, 32, ctx)
            worst = lib.pkv_attn_decode_workspace_size(batch, 32, ctx, 128)
            assert exact <= worst
    # bf16, 4 requests x 8192 keys, 8 KV heads: the stream split over 512 workgroups ((512 + 32 pairs) x G rows of
    # head_dim + 2 floats)
    p = _pool(num_kv_heads=8, num_shards=1)
    assert lib.pkv_attn_decode_workspace_size_for(C.byref(p), 4, 32, 8192) == (512 + 32) * 4 * 130 * 4
    assert lib.pkv_attn_decode_workspace_size_for(C.byref(p), 4, 30, 8192) == 0      # heads not a multiple
    assert lib.pkv_attn_decode_workspace_size_for(None, 4, 32, 8192) == 0


# ---- run_mux_round's host validation (pkv_mux_check_*: the same checks, no device) ----

def _layers(n, **kw_last):
    """n pool layers of one shape (fake aligned addresses; nothing is dereferenced), the last one altered."""
    arr = (lib_mod.PoolLayer * n)()
    for i in range(n):
        p = _pool()
        for s in range(4):
            p.k[s] = 0x100000 * (i + 1) + 0x10000 * s
            p.v[s] = 0x100000 * (i + 1) + 0x10000 * (s + 8)
        if i == n - 1:
            for k, v in kw_last.items():
                setattr(p, k, v)
        arr[i] = p
    return arr


def _ptrs(n, base, misalign_last=False):
    a = (C.c_void_p * n)()
    for i in range(n):
        a[i] = base + 0x1000 * i + (8 if misalign_last and i == n - 1 else 0)
    return a


def _decode_step(n=3, pool_kw=None, misalign=None, **kw):
    pools = _layers(n, **(pool_kw or {}))
    arrs = {k: _ptrs(n, base, misalign == k) for k, base in (("q", 0x1000000), ("k_new", 0x2000000),
                                                             ("v_new", 0x3000000), ("out", 0x4000000))}
    d = lib_mod.DecodeStep(n, C.cast(pools, C.POINTER(lib_mod.PoolLayer)),
                           *[C.cast(arrs[k], C.POINTER(C.c_void_p)) for k in ("q", "k_new", "v_new", "out")],
                           0x5000000, 0x6000000, 8, 0x7000000, 2, 64, 32, 0.0, 0x8000000, 1 << 20)
    for k, v in kw.items():
        setattr(d, k, v)
    return d, (pools, arrs)


def _prefill_job(n=3, pool_kw=None, misalign=None, **kw):
    pools = _layers(n, **(pool_kw or {}))
    arrs = {k: _ptrs(n, base, misalign == k) for k, base in (("q", 0x1000000), ("k", 0x2000000), ("v", 0x3000000),
                                                             ("out", 0x4000000))}
    p = lib_mod.PrefillJob(n, C.cast(pools, C.POINTER(lib_mod.PoolLayer)),
                           *[C.cast(arrs[k], C.POINTER(C.c_void_p)) for k in ("q", "k", "v", "out")],
                           0x5000000, 0x6000000, 8, 0x7000000, 0x7100000, 100, 32, 0.0, 0, 0)
    for k, v in kw.items():
        setattr(p, k, v)
    return p, (pools, arrs)


def test_mux_decode_step_validation():
    lib = _lib()
    ok, keep = _decode_step()
    assert lib.pkv_mux_check_decode_step(C.byref(ok)) == 0, _err(lib)
    bad = [
        _decode_step(pool_kw={"head_dim": 64}),        # a later layer with another head dim
        _decode_step(pool_kw={"dtype": lib_mod.F32}),  # ... another dtype
        _decode_step(pool_kw={"num_kv_heads": 4}),     # ... other KV heads
        _decode_step(pool_kw={"block_size": 32}),      # ... another block size
        _decode_step(pool_kw={"num_blocks": 4}),       # ... another pool size
        _decode_step(num_q_heads=30),                  # heads not a multiple of the KV heads
        _decode_step(num_q_heads=8 * 32),              # 32 q-heads per KV head: unsupported
        _decode_step(scale=float("nan")),
        _decode_step(scale=-1.0),
        _decode_step(misalign="q"), _decode_step(misalign="k_new"), _decode_step(misalign="v_new"),
        _decode_step(misalign="out"),
        _decode_step(bt_stride=2),                     # 2 blocks x 16 < 64 keys
        _decode_step(workspace=0x8000008),             # misaligned workspace (needed at 4 x 8192)
        _decode_step(workspace_bytes=16),
    ]
    bad[-2][0].batch = bad[-1][0].batch = 4
    bad[-2][0].max_context_len = bad[-1][0].max_context_len = 8192
    bad[-2][0].bt_stride = bad[-1][0].bt_stride = 512
    for d, _ in bad:
        rc = lib.pkv_mux_check_decode_step(C.byref(d))
        assert rc in (-1, -2), (rc, _err(lib))
        assert _err(lib)
    assert "layer 2" in (lib.pkv_mux_check_decode_step(C.byref(bad[0][0])), _err(lib))[1]


def test_mux_prefill_job_validation():
    lib = _lib()
    ok, keep = _prefill_job()
    assert lib.pkv_mux_check_prefill_job(C.byref(ok)) == 0, _err(lib)
    bad = [
        _prefill_job(pool_kw={"head_dim": 64}), _prefill_job(pool_kw={"dtype": lib_mod.F32}),
        _prefill_job(pool_kw={"num_shards": 2}), _prefill_job(num_q_heads=30), _prefill_job(scale=float("inf")),
        _prefill_job(misalign="q"), _prefill_job(misalign="k"), _prefill_job(misalign="v"),
        _prefill_job(misalign="out"), _prefill_job(num_tokens=200),   # 8 blocks x 16 < 200 tokens
        _prefill_job(next_layer=4),
    ]
    for p, _ in bad:
        rc = lib.pkv_mux_check_prefill_job(C.byref(p))
        assert rc in (-1, -2), (rc, _err(lib))
    assert lib.pkv_mux_check_prefill_job(None) == -1


def _mask(words):
    return (C.c_uint32 * len(words))(*words)


def test_cu_masks_keep_every_xcd():
    # [MUX] "Green contexts": a split gives decode some CUs and prefill the rest; on MI355X bit i of a mask is
    # CU i // 8 of XCD i % 8, so each queue must keep CUs on all 8 XCDs
    lib = _lib()
    for dec in (32, 48, 64, 128, 248):
        pm, dm = (C.c_uint32 * 8)(), (C.c_uint32 * 8)()
        assert lib.pkv_mux_policy_cu_masks(256, dec, pm, dm, 8) == 0
        pw, dw = list(pm), list(dm)
        assert sum(bin(w).count("1") for w in dw) == dec and sum(bin(w).count("1") for w in pw) == 256 - dec
        assert all((a & b) == 0 for a, b in zip(pw, dw)) and all((a | b) == 0xFFFFFFFF for a, b in zip(pw, dw))
        for words in (pw, dw):
            per_xcd = [sum((words[i // 32] >> (i % 32)) & 1 for i in range(256) if i % 8 == x) for x in range(8)]
            assert len(set(per_xcd)) == 1                 # the same count on every XCD
            assert lib.pkv_mux_policy_mask_ok(_mask(words), 8, 256) == 1
    # decode CUs must be a positive multiple of 8 below the total
    pm, dm = (C.c_uint32 * 8)(), (C.c_uint32 * 8)()
    for dec in (0, 4, 12, 256):
        assert lib.pkv_mux_policy_cu_masks(256, dec, pm, dm, 8) == -1


def test_mask_leaving_an_xcd_without_a_cu_is_refused():
    lib = _lib()
    # bits 0..6 of every byte-lane: XCDs 0..6 only (XCD 7 = bits 7, 15, 23, ... left out)
    no_xcd7 = [0x7F7F7F7F] * 8
    assert lib.pkv_mux_policy_mask_ok(_mask(no_xcd7), 8, 256) == 0
    # one CU on each XCD (bits 0..7) is enough
    assert lib.pkv_mux_policy_mask_ok(_mask([0xFF] + [0] * 7), 8, 256) == 1
    # seven of eight: bits 0..6
    assert lib.pkv_mux_policy_mask_ok(_mask([0x7F] + [0] * 7), 8, 256) == 0
    assert lib.pkv_mux_policy_mask_ok(_mask([0] * 8), 8, 256) == 0
    assert lib.pkv_mux_policy_mask_ok(None, 8, 256) == -1
