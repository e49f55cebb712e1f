"""Oracle for the per-layer n-gram embedding (PLE) lookup path.

TEST INFRASTRUCTURE ONLY: the plain, slow, single-threaded CPU statement of
what the path computes (C in ``ple_oracle.c``, compiled with gcc, no HIP).
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library shares no code with it and never calls
it.  Each function cites the page passage it follows in ``ple_oracle.h``.

The wrappers below marshal numpy arrays; ``prefill`` runs the stages in the
order the pages give them (ids, row lookup, merged kv_proj, gate, conv).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libple_oracle.so")


def build(force: bool = True) -> str:
    src = os.path.join(_HERE, "ple_oracle.c")
    hdr = os.path.join(_HERE, "ple_oracle.h")
    stale = (not os.path.exists(_LIB_PATH) or
             os.path.getmtime(_LIB_PATH) < max(os.path.getmtime(src), os.path.getmtime(hdr)))
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


@lru_cache(maxsize=1)
def _lib():
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_ngram_ids.argtypes = [P, P, I64, I32, P, I32, I32, I32, I32, I32, P, P, P, P, P]
    lib.orc_ngram_ids.restype = ctypes.c_int
    lib.orc_gather_bf16.argtypes = [P, I32, P, I64, P]
    lib.orc_gather_fp8.argtypes = [P, P, I32, P, I64, P]
    lib.orc_gather_fp8_global.argtypes = [P, ctypes.c_float, I32, P, I64, P]
    lib.orc_gather_nvfp4.argtypes = [P, P, ctypes.c_float, I32, P, I64, P]
    lib.orc_select_rows.argtypes = [P, I32, I64, I32, I64, I32, P]
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1_value.restype = D
    lib.orc_e4m3fn_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3fn_value.restype = D
    lib.orc_bf16_from_double.argtypes = [D]
    lib.orc_bf16_from_double.restype = ctypes.c_uint16
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = D
    lib.orc_kv_proj.argtypes = [P, P, I64, I32, I32, P]
    lib.orc_gate.argtypes = [P, P, I64, I32, D, P, P]
    lib.orc_conv.argtypes = [P, P, I64, I32, P, P, I32, I32, I32, P, P]
    lib.orc_conv.restype = ctypes.c_int
    return lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle takes C-contiguous numpy arrays"
    return a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def ngram_ids(input_ids, qsl, multipliers, vocab_sizes, offsets, *, context_len, heads_per_ngram,
              eos_token_id, ngram_context=None, first_head=0, num_heads=None, want_context_out=False):
    """IDs int32 [T, H] (and the carried context [R, C] if asked)."""
    tok = _c(input_ids, np.int32)
    q = _c(qsl, np.int32)
    mult = _c(multipliers, np.int64)
    V = _c(vocab_sizes, np.int64)
    off = _c(offsets, np.int64)
    ctx = _c(ngram_context, np.int32)
    H = len(V) if num_heads is None else num_heads
    T, R = tok.shape[0], q.shape[0] - 1
    assert mult.shape == (H, context_len + 1)
    ids = np.empty((T, H), dtype=np.int32)
    ctx_out = np.empty((R, context_len), dtype=np.int32) if want_context_out else None
    rc = _lib().orc_ngram_ids(_p(tok), _p(q), T, R, _p(ctx), context_len, heads_per_ngram, first_head, H,
                              eos_token_id, _p(mult), _p(V), _p(off), _p(ids), _p(ctx_out))
    if rc:
        raise ValueError("oracle ngram_ids: argument out of range")
    return (ids, ctx_out) if want_context_out else ids


def gather_bf16(table, ids):
    """rows [n, D] (bf16 bits) = table[ids]."""
    ids = _c(ids, np.int32).reshape(-1)
    D = table.shape[1]
    rows = np.empty((ids.shape[0], D), dtype=np.uint16)
    _lib().orc_gather_bf16(_p(table), D, _p(ids), ids.shape[0], _p(rows))
    return rows


def gather_fp8(codes, scales, ids):
    ids = _c(ids, np.int32).reshape(-1)
    D = codes.shape[1]
    rows = np.empty((ids.shape[0], D), dtype=np.uint16)
    _lib().orc_gather_fp8(_p(codes), _p(scales), D, _p(ids), ids.shape[0], _p(rows))
    return rows


def gather_fp8_global(codes, scale, ids):
    """rows [n, D] (bf16 bits) from fp8 codes with one fp32 scale for the table."""
    ids = _c(ids, np.int32).reshape(-1)
    codes = _c(codes, np.uint8)
    D = codes.shape[1]
    rows = np.empty((ids.shape[0], D), dtype=np.uint16)
    _lib().orc_gather_fp8_global(_p(codes), float(np.float32(scale)), D, _p(ids), ids.shape[0], _p(rows))
    return rows


def gather_nvfp4(codes, block_scales, tensor_scale, ids):
    """rows [n, D] (bf16 bits) from NVFP4 codes [rows, D/2], e4m3fn block scales [rows, D/16]."""
    ids = _c(ids, np.int32).reshape(-1)
    codes = _c(codes, np.uint8)
    bs = _c(block_scales, np.uint8)
    D = codes.shape[1] * 2
    assert bs.shape == (codes.shape[0], D // 16)
    rows = np.empty((ids.shape[0], D), dtype=np.uint16)
    _lib().orc_gather_nvfp4(_p(codes), _p(bs), float(np.float32(tensor_scale)), D, _p(ids), ids.shape[0], _p(rows))
    return rows


def dp_gather_slot(token_counts, group_size, dp_rank):
    """[P1] 关键源码片段 _get_dp_gather_slot: a group of group_size consecutive DP
    ranks gathers its IDs into slots of the group's largest token count; a
    rank's tokens start at (its rank within the group) * slot.  (The page
    takes the rank in the whole DP group; with one group spanning the DP group
    the two agree.)  group_size 1: (own count, 0)."""
    counts = [int(c) for c in token_counts]
    if group_size == 1:
        return counts[dp_rank], 0
    g0 = (dp_rank // group_size) * group_size
    slot = max(counts[g0:g0 + group_size])
    return slot, (dp_rank - g0) * slot


def head_shard(num_heads, tp_size, tp_rank, dp_size, dp_rank):
    """[P2] 实现拆解 item 3 (engram_head_shard_rank, TP-major): shard index
    tp_rank * dp_size + dp_rank, heads split evenly; uneven or empty shards
    are rejected (None)."""
    shards = tp_size * dp_size
    if num_heads % shards != 0 or num_heads // shards == 0:
        return None
    per = num_heads // shards
    s = tp_rank * dp_size + dp_rank
    return s * per, per


def select_rows(gathered, rank, n):
    """gathered uint16 [E][E*slot][W] -> [n][E*W] (see orc_select_rows)."""
    g = _c(gathered, np.uint16)
    E, rows, W = g.shape
    out = np.empty((n, E * W), dtype=np.uint16)
    _lib().orc_select_rows(_p(g), E, rows // E, rank, n, W, _p(out))
    return out


def e2m1_value(code: int) -> float:
    return _lib().orc_e2m1_value(code)


def e4m3fn_value(code: int) -> float:
    return _lib().orc_e4m3fn_value(code)


def bf16_from_double(x: float) -> int:
    return _lib().orc_bf16_from_double(x)


def bf16_value(bits: int) -> float:
    return _lib().orc_bf16_value(bits)


def kv_proj(x, w):
    """kv [T, O] (bf16 bits) = bf16(x @ w.T) with double accumulation."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    T, K = x.shape
    O = w.shape[0]
    assert w.shape[1] == K
    kv = np.empty((T, O), dtype=np.uint16)
    _lib().orc_kv_proj(_p(x), _p(w), T, K, O, _p(kv))
    return kv


def gate(hidden, kv, eps=1e-6):
    """(out [T, N] bf16 bits, g [T] float64)."""
    hidden = _c(hidden, np.uint16)
    kv = _c(kv, np.uint16)
    T, N = hidden.shape
    assert kv.shape == (T, 2 * N)
    out = np.empty((T, N), dtype=np.uint16)
    g = np.empty((T,), dtype=np.float64)
    _lib().orc_gate(_p(hidden), _p(kv), T, N, eps, _p(out), _p(g))
    return out, g


def conv(x, qsl, w, dilation, state=None, want_state_out=False):
    """y [T, N] (bf16 bits) and optionally the carried state [R, S, N]."""
    x = _c(x, np.uint16)
    q = _c(qsl, np.int32)
    w = _c(w, np.uint16)
    st = _c(state, np.uint16)
    T, N = x.shape
    K = w.shape[1]
    R = q.shape[0] - 1
    S = (K - 1) * dilation
    y = np.empty((T, N), dtype=np.uint16)
    so = np.empty((R, S, N), dtype=np.uint16) if want_state_out else None
    rc = _lib().orc_conv(_p(x), _p(q), T, R, _p(st), _p(w), N, K, dilation, _p(y), _p(so))
    if rc:
        raise ValueError("oracle conv: argument out of range")
    return (y, so) if want_state_out else y


def spec_commit(input_ids, x, qsl, accepted, *, conv_kernel, dilation, conv_state=None, hash_args=None,
                ngram_context=None):
    """Carried state after a speculative verify step ("Fuse Qwen4Exp PLE kernels",
    实现拆解 items 4-5: the conv's speculative variant and the short-conv state).

    Request r's window is [qsl[r], qsl[r+1]); only its first accepted[r] tokens
    (clamped to 0..window length) are kept.  By definition the committed state
    is the state the plain path leaves when run on the batch that holds only the
    kept tokens, so this builds that batch and calls ``conv`` and
    ``ngram_ids`` on it.  Returns (conv_state_out [R, S, N] or None,
    ngram_context_out [R, C] or None); x is None skips the conv part and
    hash_args (the keyword arguments of ``ngram_ids`` other than the batch) None
    skips the context part.
    """
    q = np.asarray(qsl, dtype=np.int64)
    R = q.shape[0] - 1
    keep = []
    new_q = [0]
    for r in range(R):
        a, b = int(q[r]), int(q[r + 1])
        acc = min(max(int(accepted[r]), 0), b - a)
        keep.extend(range(a, a + acc))
        new_q.append(new_q[-1] + acc)
    keep = np.asarray(keep, dtype=np.int64)
    new_q = np.asarray(new_q, dtype=np.int32)
    state_out = ctx_out = None
    if x is not None:
        x = np.asarray(x, dtype=np.uint16)
        N = x.shape[1]
        w = np.zeros((N, conv_kernel), dtype=np.uint16)
        _, state_out = conv(x[keep].reshape(-1, N), new_q, w, dilation, state=conv_state, want_state_out=True)
    if hash_args is not None:
        tok = np.asarray(input_ids, dtype=np.int32)[keep]
        _, ctx_out = ngram_ids(tok, new_q, ngram_context=ngram_context, want_context_out=True, **hash_args)
    return state_out, ctx_out


def prefill(batch_ids_args: dict, table, scales, hidden, kv_weight, conv_weight, dilation, *,
            qsl, eps=1e-6, conv_state=None, tokens=None):
    """Whole path: ids -> rows -> kv -> gate -> conv.

    ``tokens`` (optional, sorted) restricts the row gather and kv_proj to the
    listed tokens and the conv taps they need; outputs at other tokens are then
    meaningless, and the caller compares only the listed ones.  Returns a dict
    of every stage.
    """
    ids = ngram_ids(**batch_ids_args)
    T, H = ids.shape

    def gather(sel):
        if scales is None:
            return gather_bf16(table, sel)
        if isinstance(scales, tuple):  # NVFP4: (block_scales, tensor_scale)
            return gather_nvfp4(table, scales[0], scales[1], sel)
        if np.size(scales) == 1 and table.shape[0] != 1:
            return gather_fp8_global(table, np.asarray(scales).reshape(-1)[0], sel)
        return gather_fp8(table, scales, sel)

    if tokens is None:
        rows = gather(ids).reshape(T, -1)
        kv = kv_proj(rows, kv_weight)
    else:
        need = conv_taps(tokens, qsl, conv_weight.shape[1], dilation)
        D = table.shape[1] * (2 if isinstance(scales, tuple) else 1)
        rows = np.zeros((T, H * D), dtype=np.uint16)
        rows[need] = gather(ids[need]).reshape(len(need), -1)
        kv = np.zeros((T, kv_weight.shape[0]), dtype=np.uint16)
        kv[need] = kv_proj(rows[need], kv_weight)
    out, g = gate(hidden, kv, eps)
    y = conv(out, qsl, conv_weight, dilation, state=conv_state)
    return {"ids": ids, "rows": rows, "kv": kv, "gated": out, "gate": g, "y": y}


def conv_taps(tokens, qsl, kernel, dilation):
    """Sorted token indices that the conv outputs at `tokens` read (same request only)."""
    q = np.asarray(qsl, dtype=np.int64)
    need = set()
    for t in np.asarray(tokens, dtype=np.int64):
        r = int(np.searchsorted(q, t, side="right") - 1)
        for i in range(kernel):
            p = int(t) - i * dilation
            if p >= q[r]:
                need.add(p)
    return np.asarray(sorted(need), dtype=np.int64)
