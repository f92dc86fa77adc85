"""attn_decode_noalloc: attn_decode with the split partials in the library's fixed device scratch.

For callers that cannot allocate.  The GPU test runs the entry point through the C ABI twice in a row (the second
call with a smaller input, so the scratch holds the first call's rows when the second starts) and compares each
output with attn_decode's on a caller workspace (the same kernels and plan: bit for bit) and with the oracle
(bf16: max |err| <= 2e-2, rel-L2 <= 5e-3).  The CPU tests check the host-side limit and argument checks.
"""

import ctypes as C

import numpy as np
import pytest
import torch

from decode_paged_kv_amd import _lib, inputs, ops

lib_mod = _lib


def _lib_or_skip():
    try:
        return _lib.load()
    except Exception as e:  # noqa: BLE001
        pytest.skip(f"libpkv not built: {e}")


def _fake_pool(dtype, hkv=8, head_dim=128, blocks=8):
    p = lib_mod.PoolLayer()
    p.num_blocks, p.block_size, p.num_kv_heads, p.num_shards, p.head_dim = blocks, 16, hkv, 1, head_dim
    p.dtype = dtype
    p.k[0], p.v[0] = 0x100000, 0x200000
    return p


def test_noalloc_rejects_a_plan_beyond_its_scratch():
    # fp32, 63 requests x 8 KV heads (504 pairs, below one workgroup per pair), contexts up to 65536: equal splits
    # of 512 keys need 63 x 64 x 128 x 130 x 4 B of partials, far above 16 MiB
    lib = _lib_or_skip()
    p = _fake_pool(lib_mod.F32, blocks=4096)
    need = lib.pkv_attn_decode_workspace_size_for(C.byref(p), 63, 64, 65536)
    assert need > (16 << 20)
    rc = lib.attn_decode_noalloc(C.byref(p), 0x1000, 0x2000, 0x3000, 4096, 0x4000, 63, 65536, 64, 0.0, None)
    assert rc == -4 and "scratch" in lib.pkv_last_error().decode()


def test_noalloc_host_checks_as_attn_decode():
    lib = _lib_or_skip()
    p = _fake_pool(lib_mod.BF16)
    call = lambda **kw: lib.attn_decode_noalloc(  # noqa: E731
        C.byref(p), kw.get("q", 0x1000), 0x2000, 0x3000, kw.get("bt_stride", 8), 0x4000, kw.get("batch", 2),
        kw.get("max_ctx", 64), kw.get("hq", 32), kw.get("scale", 0.0), None)
    assert call(q=0x1008) == -1                      # misaligned q
    assert call(bt_stride=2) == -1                   # 2 blocks x 16 < 64 keys
    assert call(hq=30) == -1                         # heads not a multiple of the KV heads
    assert call(scale=float("nan")) == -1
    assert call(batch=0) == 0                        # nothing to do, nothing touched




def _scenario(lengths, seed):
    from gpu_common import Scenario
    sc = Scenario(num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", lengths=lengths,
                  pool_blocks=sum(-(-n // 16) for n in lengths) + 4, scale=0.5, seed=seed)
    sc.write_all()
    return sc


@pytest.mark.gpu
def test_noalloc_matches_attn_decode_on_two_calls_in_a_row():
    from gpu_common import assert_close, from_dev, i32, to_dev
    from oracle import attention as oa
    # first: the stream split with a large partial set; second: fewer, shorter requests (smaller input)
    for lengths, seed in (([2048, 8192, 3001, 4097, 6000, 33], 81), ([700, 33, 1500], 82)):
        print(f"attn_decode_noalloc lengths={lengths}", flush=True)
        sc = _scenario(lengths, seed)
        b = len(lengths)
        q = inputs.normal((b, 64, 128), 0.5, "bf16", inputs.stream(seed, 0, 0, inputs.T_Q))
        qd = to_dev(q, "bf16")
        ctx = i32(lengths)
        assert ops.attn_decode_workspace_size_for(sc.pool, b, 64, max(lengths)) > 0      # the scratch is used
        ref_out = torch.empty((b, 64, 128), dtype=torch.bfloat16, device="cuda")
        ops.attn_decode(sc.pool, qd, ref_out, sc.bt_dev, ctx, max(lengths), 64)
        out = torch.full((b, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        ops.attn_decode_noalloc(sc.pool, qd, out, sc.bt_dev, ctx, max(lengths), 64)
        torch.cuda.synchronize()
        got, want = from_dev(out, "bf16"), from_dev(ref_out, "bf16")
        assert np.array_equal(got, want), "attn_decode_noalloc differs from attn_decode"
        qf = inputs.as_float(q, "bf16")
        ref = np.stack([oa.decode(qf[r], sc.kf(r), sc.vf(r)) for r in range(b)])
        assert_close(inputs.as_float(got, "bf16"), ref, "bf16", f"attn_decode_noalloc {lengths}")
