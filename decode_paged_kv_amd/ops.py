"""Python binding of libpkv with the C ABI's names.

Only argument marshalling happens here: torch supplies device memory and
streams, every step of the path runs in the library's HIP kernels, and a
failed call raises ``PkvError`` with the library's message.  There is no
CPU fallback; without ``libpkv.so`` every call raises ``PkvLibraryMissing``.
"""

from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._lib import BF16, F32, FP8_E4M3, DecodeStep, KvDest, PkvError, PkvLibraryMissing, PoolLayer, PrefillJob  # noqa: F401
from ._lib import LAYOUT_KV_FUSED, LAYOUT_POOL, LAYOUT_TOKEN_MAJOR  # noqa: F401
from ._lib import ERRBIT_BLOCK_ID, ERRBIT_CONTEXT, ERRBIT_SLOT, ERRBIT_TABLE  # noqa: F401

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_CODE = {"bf16": BF16, "f32": F32}


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class PagedPool:
    """One layer of one instance's KV pool, in the library's layout.

    Shard ``s`` holds KV heads ``[s*H/S, (s+1)*H/S)``:
    ``k[s]`` is ``[num_blocks, H/S, block_size, head_dim]`` and ``v[s]`` is
    ``[num_blocks, H/S, head_dim, block_size]``.
    """

    def __init__(self, num_blocks, block_size, num_kv_heads, num_shards, head_dim, dtype="bf16",
                 device="cuda", err_word=None, k=None, v=None):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.num_shards, self.head_dim = num_kv_heads, num_shards, head_dim
        self.dtype = dtype
        hl = num_kv_heads // num_shards
        td = _TORCH_DTYPE[dtype]
        self.k = k if k is not None else [torch.empty((num_blocks, hl, block_size, head_dim), dtype=td, device=device)
                                          for _ in range(num_shards)]
        self.v = v if v is not None else [torch.empty((num_blocks, hl, head_dim, block_size), dtype=td, device=device)
                                          for _ in range(num_shards)]
        self.err_word = err_word

    def set_err_word(self, err_word) -> None:
        self.err_word = err_word
        self._c = None

    def fill_bits(self, pattern: int) -> "PagedPool":
        """Fill every element with one raw bit pattern (16-bit for bf16, 32-bit for f32)."""
        for t in self.k + self.v:
            (t.view(torch.int16) if self.dtype == "bf16" else t.view(torch.int32)).fill_(pattern)
        return self

    def c(self) -> PoolLayer:
        """The C descriptor (built once; the pool's tensors never change)."""
        if getattr(self, "_c", None) is None:
            self._c = self._build_c()
        return self._c

    def _build_c(self) -> PoolLayer:
        s = PoolLayer()
        for i in range(self.num_shards):
            s.k[i] = self.k[i].data_ptr()
            s.v[i] = self.v[i].data_ptr()
        s.num_blocks, s.block_size = self.num_blocks, self.block_size
        s.num_kv_heads, s.num_shards, s.head_dim = self.num_kv_heads, self.num_shards, self.head_dim
        s.dtype = _CODE[self.dtype]
        s.err_word = _ptr(self.err_word)
        return s


def slot_mapping(block_tables, start_loc, pos_start, num_tokens, block_size, num_blocks, out=None,
                 err_word=None, stream=None):
    lib = _lib.load()
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int32, device=block_tables.device)
    batch = start_loc.numel() - 1
    rc = lib.pkv_slot_mapping(_ptr(block_tables), block_tables.shape[-1], _ptr(start_loc), _ptr(pos_start), batch,
                              num_tokens, block_size, num_blocks, _ptr(out), _ptr(err_word), _stream(stream))
    _lib.check(rc, "pkv_slot_mapping")
    return out


def kv_write(pool: PagedPool, k, v, slots, stream=None):
    lib = _lib.load()
    _lib.check(lib.kv_write(C.byref(pool.c()), _ptr(k), _ptr(v), _ptr(slots), slots.numel(), _stream(stream)),
               "kv_write")


def kv_relayout(src: PagedPool, src_bt, dst: PagedPool, dst_bt, n_tokens: int, stream=None):
    lib = _lib.load()
    _lib.check(lib.kv_relayout(C.byref(src.c()), _ptr(src_bt), C.byref(dst.c()), _ptr(dst_bt), n_tokens,
                               _stream(stream)), "kv_relayout")


class ConvertedPool:
    """Destination of kv_relayout_convert: one layer in another element type and/or physical layout.

    ``dtype`` is "bf16", "f32" or "fp8" (E4M3 bits, stored as uint8; values are bits x ``scale``).  Per shard:
    layout "pool" ``k[s]`` [blocks, H/S, bs, D] and ``v[s]`` [blocks, H/S, D, bs]; "token_major" ``k[s]`` and
    ``v[s]`` [blocks, bs, H/S, D]; "kv_fused" ``k[s]`` [blocks, 2, bs, H/S, D] (K then V) and no ``v``.
    """

    _LAYOUT = {"pool": LAYOUT_POOL, "token_major": LAYOUT_TOKEN_MAJOR, "kv_fused": LAYOUT_KV_FUSED}
    _TD = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}
    _DT = {"bf16": BF16, "f32": F32, "fp8": FP8_E4M3}

    def __init__(self, num_blocks, block_size, num_kv_heads, num_shards, head_dim, dtype="bf16", layout="pool",
                 scale=1.0, device="cuda"):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.num_shards, self.head_dim = num_kv_heads, num_shards, head_dim
        self.dtype, self.layout, self.scale = dtype, layout, float(scale)
        hl, td = num_kv_heads // num_shards, self._TD[dtype]
        if layout == "pool":
            ks, vs = (num_blocks, hl, block_size, head_dim), (num_blocks, hl, head_dim, block_size)
        elif layout == "token_major":
            ks = vs = (num_blocks, block_size, hl, head_dim)
        else:
            ks, vs = (num_blocks, 2, block_size, hl, head_dim), None
        self.k = [torch.empty(ks, dtype=td, device=device) for _ in range(num_shards)]
        self.v = [torch.empty(vs, dtype=td, device=device) for _ in range(num_shards)] if vs else []

    def fill_bits(self, pattern: int) -> "ConvertedPool":
        view = {"bf16": torch.int16, "f32": torch.int32, "fp8": torch.uint8}[self.dtype]
        for t in self.k + self.v:
            t.view(view).fill_(pattern)
        return self

    def c(self) -> KvDest:
        s = KvDest()
        for i in range(self.num_shards):
            s.k[i] = self.k[i].data_ptr()
            s.v[i] = self.v[i].data_ptr() if self.v else None
        s.num_blocks, s.block_size = self.num_blocks, self.block_size
        s.num_kv_heads, s.num_shards, s.head_dim = self.num_kv_heads, self.num_shards, self.head_dim
        s.dtype, s.layout, s.scale = self._DT[self.dtype], self._LAYOUT[self.layout], self.scale
        return s


def kv_relayout_convert(src: PagedPool, src_bt, dst: ConvertedPool, dst_bt, n_tokens: int, stream=None):
    lib = _lib.load()
    _lib.check(lib.kv_relayout_convert(C.byref(src.c()), _ptr(src_bt), C.byref(dst.c()), _ptr(dst_bt), n_tokens,
                                       _stream(stream)), "kv_relayout_convert")


def attn_prefill_chunk(pool: PagedPool, q, out, block_tables, start_loc, chunk_start, max_chunk_len: int,
                       num_q_heads: int, scale: float = 0.0, stream=None, max_total_len: int | None = None):
    """``max_total_len`` (an upper bound of every S+T) defaults to what the block table addresses."""
    lib = _lib.load()
    c = pool.c()
    batch = chunk_start.numel()
    if max_total_len is None:
        max_total_len = block_tables.shape[-1] * pool.block_size
    rc = lib.attn_prefill_chunk(C.byref(c), _ptr(q), _ptr(out), _ptr(block_tables), block_tables.shape[-1],
                                _ptr(start_loc), _ptr(chunk_start), batch, max_chunk_len, max_total_len, num_q_heads,
                                scale, _stream(stream))
    _lib.check(rc, "attn_prefill_chunk")


def attn_decode_workspace_size(batch: int, num_q_heads: int, max_context_len: int, head_dim: int) -> int:
    """Worst case over group sizes and dtypes (the library is told neither)."""
    return int(_lib.load().pkv_attn_decode_workspace_size(batch, num_q_heads, max_context_len, head_dim))


def attn_decode_workspace_size_for(pool: PagedPool, batch: int, num_q_heads: int, max_context_len: int) -> int:
    """Exactly what attn_decode needs for this pool (KV heads, head dim, dtype)."""
    return int(_lib.load().pkv_attn_decode_workspace_size_for(C.byref(pool.c()), batch, num_q_heads,
                                                               max_context_len))


def attn_decode(pool: PagedPool, q, out, block_tables, context_lens, max_context_len: int, num_q_heads: int,
                scale: float = 0.0, workspace=None, stream=None):
    lib = _lib.load()
    c = pool.c()
    batch = context_lens.numel()
    if workspace is None:
        nbytes = attn_decode_workspace_size(batch, num_q_heads, max_context_len, pool.head_dim)
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = lib.attn_decode(C.byref(c), _ptr(q), _ptr(out), _ptr(block_tables), block_tables.shape[-1],
                         _ptr(context_lens), batch, max_context_len, num_q_heads, scale, _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check(rc, "attn_decode")


def attn_decode_noalloc(pool: PagedPool, q, out, block_tables, context_lens, max_context_len: int, num_q_heads: int,
                        scale: float = 0.0, stream=None):
    """attn_decode with the split partials in the library's fixed device scratch (no workspace, no allocation)."""
    lib = _lib.load()
    rc = lib.attn_decode_noalloc(C.byref(pool.c()), _ptr(q), _ptr(out), _ptr(block_tables), block_tables.shape[-1],
                                 _ptr(context_lens), context_lens.numel(), max_context_len, num_q_heads, scale,
                                 _stream(stream))
    _lib.check(rc, "attn_decode_noalloc")


def attn_decode_append(pool: PagedPool, q, k_new, v_new, out, block_tables, context_lens, max_context_len: int,
                       num_q_heads: int, scale: float = 0.0, workspace=None, stream=None):
    """kv_write of each request's new row at position L-1 and attn_decode over [0, L), in one launch."""
    lib = _lib.load()
    c = pool.c()
    batch = context_lens.numel()
    if workspace is None:
        nbytes = attn_decode_workspace_size(batch, num_q_heads, max_context_len, pool.head_dim)
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = lib.attn_decode_append(C.byref(c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(block_tables),
                                block_tables.shape[-1], _ptr(context_lens), batch, max_context_len, num_q_heads,
                                scale, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _lib.check(rc, "attn_decode_append")


def stall_free_chunk(token_budget: int, num_decode: int, prompt_remaining: int) -> int:
    """Tokens of a prompt that fit a stall-free step: what the decode requests leave of the budget."""
    rc = int(_lib.load().pkv_stall_free_chunk(token_budget, num_decode, prompt_remaining))
    _lib.check(rc if rc < 0 else 0, "pkv_stall_free_chunk")
    return rc


def stall_free_batch(token_budget: int, num_decode: int, prompts_remaining) -> list[int]:
    """Chunks of several prompts in one stall-free step (ongoing prefills listed before new requests)."""
    n = len(prompts_remaining)
    rem = (C.c_int32 * max(n, 1))(*[int(x) for x in prompts_remaining])
    out = (C.c_int32 * max(n, 1))()
    rc = int(_lib.load().pkv_stall_free_batch(token_budget, num_decode, rem, n, out))
    _lib.check(rc if rc < 0 else 0, "pkv_stall_free_batch")
    return [int(out[i]) for i in range(n)]


def attn_mixed_batch(pool: PagedPool, q_dec, out_dec, dec_block_tables, context_lens, max_context_len: int,
                     q_pf, out_pf, pf_block_tables, start_loc, chunk_start, max_chunk_len: int, num_q_heads: int,
                     scale: float = 0.0, workspace=None, stream=None, max_total_len: int | None = None):
    """Decode attention for every request in context_lens and prefill attention for the chunks described by
    start_loc / chunk_start, one launch (bf16).  Pass None for the tensors of an empty part."""
    lib = _lib.load()
    c = pool.c()
    nd = 0 if context_lens is None else context_lens.numel()
    npf = 0 if chunk_start is None else chunk_start.numel()
    if workspace is None and nd > 0:
        nbytes = attn_decode_workspace_size(nd, num_q_heads, max_context_len, pool.head_dim)
        dev = q_dec.device
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if max_total_len is None:
        max_total_len = 0 if pf_block_tables is None else pf_block_tables.shape[-1] * pool.block_size
    p = lambda t: None if t is None else _ptr(t)  # noqa: E731
    rc = lib.attn_mixed_batch(C.byref(c), p(q_dec), p(out_dec), p(dec_block_tables),
                              0 if dec_block_tables is None else dec_block_tables.shape[-1], p(context_lens), nd,
                              max_context_len, p(q_pf), p(out_pf), p(pf_block_tables),
                              0 if pf_block_tables is None else pf_block_tables.shape[-1], p(start_loc),
                              p(chunk_start), npf, max_chunk_len, max_total_len, num_q_heads, scale, p(workspace),
                              ws_bytes,
                              _stream(stream))
    _lib.check(rc, "attn_mixed_batch")


def _ptr_array(tensors):
    arr = (C.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = _ptr(t)
    return arr


def _pool_array(pools):
    arr = (PoolLayer * len(pools))()
    for i, p in enumerate(pools):
        arr[i] = p.c()
    return arr


class DecodeStepArgs:
    """Keeps the ctypes arrays of one decode step alive while it is in use."""

    def __init__(self, pools, q, k_new, v_new, out, slots, block_tables, context_lens, max_context_len,
                 num_q_heads, workspace, scale=0.0):
        self._keep = (_pool_array(pools), _ptr_array(q), _ptr_array(k_new), _ptr_array(v_new), _ptr_array(out))
        self.c = DecodeStep(len(pools), C.cast(self._keep[0], C.POINTER(PoolLayer)),
                            C.cast(self._keep[1], C.POINTER(C.c_void_p)), C.cast(self._keep[2], C.POINTER(C.c_void_p)),
                            C.cast(self._keep[3], C.POINTER(C.c_void_p)), C.cast(self._keep[4], C.POINTER(C.c_void_p)),
                            _ptr(slots), _ptr(block_tables), block_tables.shape[-1], _ptr(context_lens),
                            context_lens.numel(), max_context_len, num_q_heads, scale, _ptr(workspace),
                            workspace.numel() * workspace.element_size())
        self._tensors = (slots, block_tables, context_lens, workspace)


class PrefillJobArgs:
    """A whole-prompt, layer-by-layer prefill job; ``c.next_layer`` is the cursor."""

    def __init__(self, pools, q, k, v, out, slots, block_table, start_loc, chunk_start, num_tokens, num_q_heads,
                 scale=0.0):
        self._keep = (_pool_array(pools), _ptr_array(q), _ptr_array(k), _ptr_array(v), _ptr_array(out))
        self.c = PrefillJob(len(pools), C.cast(self._keep[0], C.POINTER(PoolLayer)),
                            C.cast(self._keep[1], C.POINTER(C.c_void_p)), C.cast(self._keep[2], C.POINTER(C.c_void_p)),
                            C.cast(self._keep[3], C.POINTER(C.c_void_p)), C.cast(self._keep[4], C.POINTER(C.c_void_p)),
                            _ptr(slots), _ptr(block_table), block_table.shape[-1], _ptr(start_loc), _ptr(chunk_start),
                            num_tokens, num_q_heads, scale, 0, 0)
        self._tensors = (slots, block_table, start_loc, chunk_start)

    @property
    def done_submitting(self) -> bool:
        return bool(self.c.submitted_all)


class Mux:
    """CU-masked stream pairs per split level and the multiplexing round loop."""

    def __init__(self, device=0, cu_granularity=8, min_decode_cus=32, sm_group_num=8, decode_bs_divisor=36,
                 token_budget=65536):
        lib = _lib.load()
        h = C.c_void_p()
        _lib.check(lib.pkv_mux_create(device, cu_granularity, min_decode_cus, sm_group_num, decode_bs_divisor,
                                      token_budget, C.byref(h)), "pkv_mux_create")
        self._h = h

    def close(self):
        if self._h:
            _lib.load().pkv_mux_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def groups(self):
        lib = _lib.load()
        cap = 64
        p, d, n = (C.c_int32 * cap)(), (C.c_int32 * cap)(), C.c_int32()
        _lib.check(lib.pkv_mux_groups(self._h, p, d, cap, C.byref(n)), "pkv_mux_groups")
        return [(p[i], d[i]) for i in range(n.value)]

    def choose(self, decode_bs: int, has_prefill: bool) -> int:
        return int(_lib.load().pkv_mux_choose(self._h, decode_bs, int(has_prefill)))

    def layers_per_round(self, prefill_tokens: int, num_layers: int) -> int:
        return int(_lib.load().pkv_mux_layers_per_round(self._h, prefill_tokens, num_layers))

    def set_level_override(self, level: int) -> None:
        _lib.check(_lib.load().pkv_mux_set_level_override(self._h, level), "pkv_mux_set_level_override")

    def set_decode_graphs(self, enable: bool) -> None:
        """Capture each level's decode step as one HIP graph and replay it while its arguments stay the same."""
        _lib.check(_lib.load().pkv_mux_set_decode_graphs(self._h, int(bool(enable))), "pkv_mux_set_decode_graphs")

    def set_decode_append(self, enable: bool) -> None:
        """Run each decode layer as one attn_decode_append (write + attention) instead of kv_write + attn_decode."""
        _lib.check(_lib.load().pkv_mux_set_decode_append(self._h, int(bool(enable))), "pkv_mux_set_decode_append")

    def set_manual_divisions(self, thresholds) -> None:
        """Decode batch size from which each split level is used (None or [] restores the divisor rule)."""
        t = list(thresholds or [])
        arr = (C.c_int32 * max(1, len(t)))(*t)
        _lib.check(_lib.load().pkv_mux_set_manual_divisions(self._h, arr, len(t)), "pkv_mux_set_manual_divisions")

    def stream(self, level: int, which: int) -> int:
        return int(_lib.load().pkv_mux_stream(self._h, level, which) or 0)

    def cu_mask(self, level: int, which: int):
        lib = _lib.load()
        words, n = (C.c_uint32 * 16)(), C.c_int32()
        _lib.check(lib.pkv_mux_cu_mask(self._h, level, which, words, 16, C.byref(n)), "pkv_mux_cu_mask")
        return [words[i] for i in range(n.value)]

    def run_round(self, decode: DecodeStepArgs | None, prefill: PrefillJobArgs | None):
        """One round; returns (level, prefill_done)."""
        lib = _lib.load()
        lvl, done = C.c_int32(), C.c_int32()
        rc = lib.run_mux_round(self._h, C.byref(decode.c) if decode else None,
                               C.byref(prefill.c) if prefill else None, C.byref(lvl), C.byref(done))
        _lib.check(rc, "run_mux_round")
        return lvl.value, bool(done.value)

    def wait_prefill(self):
        _lib.check(_lib.load().pkv_mux_wait_prefill(self._h), "pkv_mux_wait_prefill")


run_mux_round = Mux.run_round
