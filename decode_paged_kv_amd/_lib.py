"""ctypes view of libpkv's C ABI (include/pkv.h).  Marshalling only."""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB_PATH selects another build of the same library (e.g. one whose
# host code is compiled with sanitizers)
LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(HERE, "libpkv.so")

MAX_SHARDS = 16
F32, BF16, FP8_E4M3 = 0, 1, 2
LAYOUT_POOL, LAYOUT_TOKEN_MAJOR, LAYOUT_KV_FUSED = 0, 1, 2
OK, EINVAL, EUNSUPPORTED, EHIP, ERANGE = 0, -1, -2, -3, -4
ERRBIT_BLOCK_ID, ERRBIT_SLOT, ERRBIT_TABLE, ERRBIT_CONTEXT = 1, 2, 4, 8


class PkvLibraryMissing(RuntimeError):
    """libpkv.so has not been built; there is no fallback implementation."""


class PkvError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func} failed with {code}: {msg}")
        self.code = code


class PoolLayer(C.Structure):
    _fields_ = [
        ("k", C.c_void_p * MAX_SHARDS),
        ("v", C.c_void_p * MAX_SHARDS),
        ("num_blocks", C.c_int32),
        ("block_size", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("num_shards", C.c_int32),
        ("head_dim", C.c_int32),
        ("dtype", C.c_int32),
        ("err_word", C.c_void_p),
    ]


class KvDest(C.Structure):
    _fields_ = [
        ("k", C.c_void_p * MAX_SHARDS),
        ("v", C.c_void_p * MAX_SHARDS),
        ("num_blocks", C.c_int32),
        ("block_size", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("num_shards", C.c_int32),
        ("head_dim", C.c_int32),
        ("dtype", C.c_int32),
        ("layout", C.c_int32),
        ("scale", C.c_float),
    ]


class DecodeStep(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32),
        ("pools", C.POINTER(PoolLayer)),
        ("q", C.POINTER(C.c_void_p)),
        ("k_new", C.POINTER(C.c_void_p)),
        ("v_new", C.POINTER(C.c_void_p)),
        ("out", C.POINTER(C.c_void_p)),
        ("slots", C.c_void_p),
        ("block_tables", C.c_void_p),
        ("bt_stride", C.c_int32),
        ("context_lens", C.c_void_p),
        ("batch", C.c_int32),
        ("max_context_len", C.c_int32),
        ("num_q_heads", C.c_int32),
        ("scale", C.c_float),
        ("workspace", C.c_void_p),
        ("workspace_bytes", C.c_size_t),
    ]


class PrefillJob(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32),
        ("pools", C.POINTER(PoolLayer)),
        ("q", C.POINTER(C.c_void_p)),
        ("k", C.POINTER(C.c_void_p)),
        ("v", C.POINTER(C.c_void_p)),
        ("out", C.POINTER(C.c_void_p)),
        ("slots", C.c_void_p),
        ("block_table", C.c_void_p),
        ("bt_stride", C.c_int32),
        ("start_loc", C.c_void_p),
        ("chunk_start", C.c_void_p),
        ("num_tokens", C.c_int32),
        ("num_q_heads", C.c_int32),
        ("scale", C.c_float),
        ("next_layer", C.c_int32),
        ("submitted_all", C.c_int32),
    ]


_P = C.c_void_p
_I = C.c_int32
_SIGS = {
    "pkv_last_error": (C.c_char_p, []),
    "pkv_version": (C.c_int, []),
    "pkv_slot_mapping": (C.c_int, [_P, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "kv_write": (C.c_int, [C.POINTER(PoolLayer), _P, _P, _P, _I, _P]),
    "kv_relayout": (C.c_int, [C.POINTER(PoolLayer), _P, C.POINTER(PoolLayer), _P, _I, _P]),
    "kv_relayout_convert": (C.c_int, [C.POINTER(PoolLayer), _P, C.POINTER(KvDest), _P, _I, _P]),
    "attn_prefill_chunk": (C.c_int, [C.POINTER(PoolLayer), _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, C.c_float, _P]),
    "pkv_attn_decode_workspace_size": (C.c_size_t, [_I, _I, _I, _I]),
    "pkv_attn_decode_workspace_size_for": (C.c_size_t, [C.POINTER(PoolLayer), _I, _I, _I]),
    "attn_decode": (C.c_int, [C.POINTER(PoolLayer), _P, _P, _P, _I, _P, _I, _I, _I, C.c_float, _P, C.c_size_t, _P]),
    "attn_decode_append": (C.c_int, [C.POINTER(PoolLayer), _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, C.c_float, _P,
                                     C.c_size_t, _P]),
    "pkv_stall_free_chunk": (C.c_int, [_I, _I, _I]),
    "attn_mixed_batch": (C.c_int, [C.POINTER(PoolLayer), _P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _I, _P, _P, _I, _I,
                                   _I, _I, C.c_float, _P, C.c_size_t, _P]),
    "pkv_mux_policy_groups_grid": (C.c_int, [C.c_int] * 5 + [C.POINTER(_I), C.POINTER(_I), _I, C.POINTER(_I)]),
    "pkv_mux_policy_choose": (C.c_int, [C.c_int] * 4),
    "pkv_mux_policy_layers_per_round": (C.c_int, [C.c_int] * 3),
    "pkv_mux_create": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(_P)]),
    "pkv_mux_destroy": (None, [_P]),
    "pkv_mux_groups": (C.c_int, [_P, C.POINTER(_I), C.POINTER(_I), _I, C.POINTER(_I)]),
    "pkv_mux_choose": (C.c_int, [_P, C.c_int, C.c_int]),
    "pkv_mux_layers_per_round": (C.c_int, [_P, C.c_int, C.c_int]),
    "pkv_mux_set_level_override": (C.c_int, [_P, C.c_int]),
    "pkv_mux_set_manual_divisions": (C.c_int, [_P, C.POINTER(_I), _I]),
    "pkv_mux_set_decode_graphs": (C.c_int, [_P, C.c_int]),
    "pkv_mux_set_decode_append": (C.c_int, [_P, C.c_int]),
    "pkv_mux_policy_choose_manual": (C.c_int, [C.c_int, C.c_int, C.c_int, C.POINTER(_I)]),
    "pkv_mux_stream": (_P, [_P, C.c_int, C.c_int]),
    "pkv_mux_cu_mask": (C.c_int, [_P, C.c_int, C.c_int, C.POINTER(C.c_uint32), _I, C.POINTER(_I)]),
    "run_mux_round": (C.c_int, [_P, C.POINTER(DecodeStep), C.POINTER(PrefillJob), C.POINTER(_I), C.POINTER(_I)]),
    "pkv_mux_wait_prefill": (C.c_int, [_P]),
    "pkv_stall_free_batch": (C.c_int, [_I, _I, C.POINTER(_I), _I, C.POINTER(_I)]),
    "attn_decode_noalloc": (C.c_int, [C.POINTER(PoolLayer), _P, _P, _P, _I, _P, _I, _I, _I, C.c_float, _P]),
    "pkv_mux_check_decode_step": (C.c_int, [C.POINTER(DecodeStep)]),
    "pkv_mux_check_prefill_job": (C.c_int, [C.POINTER(PrefillJob)]),
    "pkv_mux_policy_cu_masks": (C.c_int, [C.c_int, C.c_int, C.POINTER(C.c_uint32), C.POINTER(C.c_uint32), _I]),
    "pkv_mux_policy_mask_ok": (C.c_int, [C.POINTER(C.c_uint32), _I, C.c_int]),
}
EXPORTED = tuple(_SIGS)

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """The loaded library (loaded once).  Raises PkvLibraryMissing if unbuilt."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise PkvLibraryMissing(
            f"{path} is not built; run `python -m decode_paged_kv_amd.build` (needs hipcc for gfx950)")
    lib = C.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(rc: int, func: str) -> None:
    if rc != OK:
        raise PkvError(rc, func, load().pkv_last_error().decode(errors="replace"))
