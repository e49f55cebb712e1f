"""ctypes view of libple's C ABI (include/ple.h): structures, prototypes, loader.

Argument marshalling only; every step of the path runs in libple's kernels.
Loading fails loudly when libple.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (load torch's HIP runtime first so libple binds to the same one)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libple.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "ple.h")

PLE_OK = 0
PLE_ERR_INVALID_ARGUMENT = 1
PLE_ERR_UNSUPPORTED = 2
PLE_ERR_DEVICE = 3
PLE_ERR_WORKSPACE = 4
PLE_DTYPE_BF16 = 0
PLE_DTYPE_FP8_E4M3 = 1
PLE_DTYPE_FP8_E4M3_GLOBAL = 2
PLE_DTYPE_NVFP4 = 3
PLE_MAX_HEADS = 32
PLE_MAX_CONTEXT = 7
PLE_NOALLOC_SCRATCH_BYTES = 64 << 20

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64


class ple_hash_desc(ctypes.Structure):
    _fields_ = [("num_heads", I32), ("heads_per_ngram", I32), ("context_len", I32), ("first_head", I32),
                ("eos_token_id", I32), ("reserved", I32),
                ("multipliers", P), ("vocab_sizes", P), ("offsets", P)]


class ple_table_desc(ctypes.Structure):
    _fields_ = [("table", P), ("num_rows", I64), ("dim", I32), ("dtype", I32), ("row_scales", P),
                ("block_scales", P)]


class ple_batch_desc(ctypes.Structure):
    _fields_ = [("input_ids", P), ("query_start_loc", P), ("num_tokens", I64), ("num_reqs", I32),
                ("max_request_tokens", I32), ("ngram_context", P), ("ngram_context_out", P),
                ("conv_state", P), ("conv_state_out", P)]


class ple_layer_desc(ctypes.Structure):
    _fields_ = [("hash", ple_hash_desc), ("table", ple_table_desc), ("kv_weight", P), ("hidden", I32),
                ("eps", ctypes.c_float), ("conv_weight", P), ("conv_kernel", I32), ("conv_dilation", I32)]


_PROTOS = {
    "ple_ngram_ids": (ctypes.c_int, [ctypes.POINTER(ple_hash_desc), ctypes.POINTER(ple_batch_desc), P, P]),
    "ple_gather": (ctypes.c_int, [ctypes.POINTER(ple_table_desc), P, I64, I32, P, P]),
    "ple_lookup": (ctypes.c_int, [ctypes.POINTER(ple_hash_desc), ctypes.POINTER(ple_table_desc),
                                  ctypes.POINTER(ple_batch_desc), P, P, P]),
    "ple_prefetch": (ctypes.c_int, [ctypes.POINTER(ple_layer_desc), ctypes.POINTER(ple_batch_desc), P, P]),
    "ple_prefetch_dedup": (ctypes.c_int, [ctypes.POINTER(ple_layer_desc), ctypes.POINTER(ple_batch_desc), P, P,
                                          ctypes.c_size_t, P, P]),
    "ple_prefetch_dedup_workspace_bytes": (ctypes.c_size_t, [I64, I32]),
    "ple_prefetch_dedup_plan": (ctypes.c_int, [ctypes.POINTER(ple_layer_desc), ctypes.POINTER(ple_batch_desc), P,
                                               ctypes.c_size_t, P]),
    "ple_prefetch_dedup_fetch": (ctypes.c_int, [ctypes.POINTER(ple_layer_desc), I64, P, ctypes.c_size_t, P, P, P]),
    "ple_dp_gather_slot": (ctypes.c_int, [P, I32, I32, I32, P, P]),
    "ple_head_shard": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P]),
    "ple_select_rows": (ctypes.c_int, [P, I32, I64, I32, I64, I32, P, P]),
    "ple_kv_proj": (ctypes.c_int, [P, P, I64, I32, I32, P, P]),
    "ple_gate": (ctypes.c_int, [P, P, I64, I32, ctypes.c_float, P, P, P]),
    "ple_conv": (ctypes.c_int, [P, ctypes.POINTER(ple_batch_desc), P, I32, I32, I32, P, P]),
    "ple_spec_commit": (ctypes.c_int, [ctypes.POINTER(ple_hash_desc), ctypes.POINTER(ple_batch_desc), P, P, I32,
                                       I32, I32, P]),
    "ple_prefill_fused": (ctypes.c_int, [ctypes.POINTER(ple_layer_desc), ctypes.POINTER(ple_batch_desc), P, P, P,
                                         P, P, ctypes.c_size_t, P]),
    "ple_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ple_layer_desc), I64]),
    "ple_prefill_fused_noalloc": (ctypes.c_int, [ctypes.POINTER(ple_layer_desc), ctypes.POINTER(ple_batch_desc), P,
                                                 P, P, P, P]),
    "ple_host_alloc": (ctypes.c_int, [ctypes.c_size_t, ctypes.POINTER(P), ctypes.POINTER(P)]),
    "ple_host_free": (ctypes.c_int, [P]),
    "ple_stream_create_cu_masked": (ctypes.c_int, [I32, ctypes.POINTER(P)]),
    "ple_stream_destroy": (ctypes.c_int, [P]),
    "ple_error_message": (ctypes.c_char_p, []),
    "ple_version": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libple.so (built in-tree).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libple.so is not built ({LIB_PATH}); run "
                               "`python -m layer_embedding_lookup_amd.build` (needs hipcc)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/ple.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ple_[a-z_0-9]+)\s*\(", text)))


def error_message() -> str:
    return load().ple_error_message().decode()


def check(rc: int, what: str) -> None:
    if rc != PLE_OK:
        raise RuntimeError(f"{what} failed (code {rc}): {error_message()}")
