"""MI355X-native per-layer n-gram embedding (PLE / Engram) lookup.

Thin Python binding over libple (include/ple.h).  The functions keep the C
names and only marshal torch tensors into the C descriptors: every step of the
path runs in libple's HIP kernels on the tensors' device, on the current torch
stream unless a stream is given.  PyTorch provides device memory and streams.

    hp = HashParams(multipliers, vocab_sizes, offsets, heads_per_ngram=4, context_len=2, eos_token_id=0)
    tb = Table.from_tensor(table)                 # bf16 [rows, D] or uint8 codes + fp32 scales
    rows = ple_lookup(hp, tb, input_ids, query_start_loc)
    kv = ple_kv_proj(rows, kv_weight)
    out, g = ple_gate(hidden, kv)
    y = ple_conv(out, query_start_loc, conv_weight, dilation=3)

Errors raise RuntimeError with the library's message.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import capi
from .capi import (PLE_DTYPE_BF16, PLE_DTYPE_FP8_E4M3, PLE_DTYPE_FP8_E4M3_GLOBAL, PLE_DTYPE_NVFP4,  # noqa: F401
                   PLE_ERR_DEVICE, PLE_ERR_INVALID_ARGUMENT,
                   PLE_ERR_UNSUPPORTED, PLE_ERR_WORKSPACE, PLE_MAX_CONTEXT, PLE_MAX_HEADS, PLE_OK)

__all__ = ["HashParams", "Table", "Layer", "ple_ngram_ids", "ple_gather", "ple_lookup", "ple_prefetch",
           "ple_prefetch_dedup", "ple_prefetch_dedup_workspace_bytes", "ple_prefetch_dedup_plan",
           "ple_prefetch_dedup_fetch", "ple_dp_gather_slot", "ple_head_shard",
           "ple_select_rows",
           "ple_kv_proj", "ple_gate", "ple_conv", "ple_spec_commit", "ple_prefill_fused", "ple_prefill_workspace_bytes",
           "ple_prefill_fused_noalloc",
           "prefill_conv_input", "prefill_kv",
           "ple_host_alloc", "ple_host_free", "HostBuffer", "ple_stream_create_cu_masked", "ple_stream_destroy",
           "ple_error_message", "ple_version", "library"]


def library() -> ctypes.CDLL:
    return capi.load()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


# Host-side checks of the tensors behind the pointers, run before any library
# call: a mismatched shape would otherwise become an out-of-bounds device
# access.  Raw integer addresses are passed through unchecked (the caller
# vouches for them).
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)
_F32 = (torch.float32,)
_BYTES = (torch.uint8, torch.int8)


def _req(name: str, t, shape, dtypes, *, optional: bool = False):
    """Check one tensor argument: dtype, exact shape (None = any size on that
    axis), contiguity.  Returns the tensor."""
    # fast path (these checks run on every call, and decode-sized calls are
    # launch-bound): a well-formed tensor passes with a few attribute reads
    if type(t) is torch.Tensor and t.dtype in dtypes:
        ts = t.shape
        if len(ts) == len(shape) and t.is_contiguous():
            for got, want in zip(ts, shape):
                if want is not None and got != want:
                    break
            else:
                return t
    return _req_checked(name, t, shape, dtypes, optional)


def _req_checked(name: str, t, shape, dtypes, optional: bool):
    """_req for anything the fast path did not pass: raises the precise error."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if len(t.shape) != len(shape) or any(want is not None and int(got) != int(want)
                                         for got, want in zip(t.shape, shape)):
        want = ", ".join("*" if w is None else str(int(w)) for w in shape)
        want = f"({want},)" if len(shape) == 1 else f"({want})"
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _req_bytes(name: str, t, nbytes: int):
    """A workspace: a contiguous byte tensor of at least nbytes."""
    if isinstance(t, int):
        return t
    _req(name, t, (None,), _BYTES)
    if t.numel() < nbytes:
        raise ValueError(f"{name} holds {t.numel()} bytes, {nbytes} needed")
    return t


def _same_device(*tensors):
    """Every tensor argument on one GPU (raw addresses and None are skipped)."""
    dev = None
    for t in tensors:
        if isinstance(t, torch.Tensor):
            d = t.get_device()  # -1 for host tensors
            if d < 0:
                raise ValueError("tensor arguments must be GPU tensors")
            if dev is None:
                dev = d
            elif d != dev:
                devs = sorted({x.get_device() for x in tensors if isinstance(x, torch.Tensor)})
                raise ValueError(f"tensor arguments are on different devices: {devs}")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class HashParams:
    """One layer's hash constants (host memory, read during each call)."""

    def __init__(self, multipliers, vocab_sizes, offsets, *, heads_per_ngram: int, context_len: int,
                 eos_token_id: int, first_head: int = 0):
        self.multipliers = np.ascontiguousarray(np.asarray(multipliers, dtype=np.int64))
        self.vocab_sizes = np.ascontiguousarray(np.asarray(vocab_sizes, dtype=np.int64))
        self.offsets = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
        self.heads_per_ngram = int(heads_per_ngram)
        self.context_len = int(context_len)
        self.eos_token_id = int(eos_token_id)
        self.first_head = int(first_head)
        self.num_heads = int(self.vocab_sizes.shape[0])

    # The C descriptor is built once and rebuilt only after an attribute is
    # reassigned (calls pass it by reference; the library only reads it).
    def __setattr__(self, key, value):
        object.__setattr__(self, key, value)
        if key != "_desc":
            object.__setattr__(self, "_desc", None)

    def desc(self) -> capi.ple_hash_desc:
        d = self._desc
        if d is None:
            d = capi.ple_hash_desc(self.num_heads, self.heads_per_ngram, self.context_len, self.first_head,
                                   self.eos_token_id, 0, self.multipliers.ctypes.data, self.vocab_sizes.ctypes.data,
                                   self.offsets.ctypes.data)
            object.__setattr__(self, "_desc", d)
        return d


class Table:
    """An embedding table: a device tensor, or the device address of mapped pinned host memory.

    `row_scales_ptr` is the per-row fp32 scales (PLE_DTYPE_FP8_E4M3) or the
    one fp32 table scale (PLE_DTYPE_FP8_E4M3_GLOBAL, PLE_DTYPE_NVFP4);
    `block_scales_ptr` the NVFP4 e4m3fn scale per 16 elements."""

    def __init__(self, ptr: int, num_rows: int, dim: int, dtype: int, row_scales_ptr: int | None = None,
                 keepalive=(), block_scales_ptr: int | None = None):
        self.ptr, self.num_rows, self.dim, self.dtype = int(ptr), int(num_rows), int(dim), int(dtype)
        self.row_scales_ptr = row_scales_ptr
        self.block_scales_ptr = block_scales_ptr
        self._keepalive = keepalive

    @classmethod
    def from_tensor(cls, table: torch.Tensor, row_scales: torch.Tensor | None = None) -> "Table":
        """bf16 [rows][D], or fp8 codes [rows][D] with fp32 scales: [rows] per row, or [1] for the table."""
        if table.dtype in (torch.bfloat16, torch.int16, torch.uint16):
            dt = PLE_DTYPE_BF16
        elif table.dtype in (torch.uint8, torch.float8_e4m3fn):
            if row_scales is None:
                raise ValueError("an fp8 table needs its scales")
            dt = PLE_DTYPE_FP8_E4M3_GLOBAL if row_scales.numel() == 1 and table.shape[0] != 1 else PLE_DTYPE_FP8_E4M3
        else:
            raise ValueError(f"unsupported table dtype {table.dtype}")
        return cls(_ptr(table), table.shape[0], table.shape[1], dt, _ptr(row_scales), (table, row_scales))

    @classmethod
    def nvfp4(cls, codes: torch.Tensor, block_scales: torch.Tensor, tensor_scale: torch.Tensor) -> "Table":
        """codes uint8 [rows][D/2] (element 2i in the low nibble of byte i), block_scales
        uint8 e4m3fn [rows][D/16], tensor_scale fp32 [1]."""
        rows, half = codes.shape
        if block_scales.shape != (rows, half // 8) or tensor_scale.numel() != 1:
            raise ValueError("NVFP4 table: block_scales must be [rows][D/16] and tensor_scale one value")
        return cls(_ptr(codes), rows, 2 * half, PLE_DTYPE_NVFP4, _ptr(tensor_scale),
                   (codes, block_scales, tensor_scale), block_scales_ptr=_ptr(block_scales))

    def __setattr__(self, key, value):
        object.__setattr__(self, key, value)
        if key != "_desc":
            object.__setattr__(self, "_desc", None)

    def desc(self) -> capi.ple_table_desc:
        d = self._desc
        if d is None:
            d = capi.ple_table_desc(self.ptr, self.num_rows, self.dim, self.dtype, self.row_scales_ptr,
                                    self.block_scales_ptr)
            object.__setattr__(self, "_desc", d)
        return d


class Layer:
    """A layer's hash, table, projection, gate and conv parameters."""

    def __init__(self, hash: HashParams, table: Table, kv_weight: torch.Tensor, conv_weight: torch.Tensor, *,
                 conv_dilation: int, eps: float = 1e-6):
        self.hash, self.table = hash, table
        _req("conv_weight", conv_weight, (None, None), _BF16)
        self.hidden = int(conv_weight.shape[0])
        self.conv_kernel = int(conv_weight.shape[1])
        _req("kv_weight", kv_weight, (2 * self.hidden, hash.num_heads * table.dim), _BF16)
        self.kv_weight, self.conv_weight = kv_weight, conv_weight
        self.conv_dilation = int(conv_dilation)
        self.eps = float(eps)

    def __setattr__(self, key, value):
        object.__setattr__(self, key, value)
        if key not in ("_desc", "_desc_parts", "_ws_bytes"):
            object.__setattr__(self, "_desc", None)

    def desc(self) -> capi.ple_layer_desc:
        """The layer's C descriptor, rebuilt when an attribute (or the hash's or
        table's descriptor) has changed; workspace sizes are cached with it."""
        hd, td = self.hash.desc(), self.table.desc()
        d = self._desc
        if d is None or self._desc_parts[0] is not hd or self._desc_parts[1] is not td:
            d = capi.ple_layer_desc(hd, td, _ptr(self.kv_weight), self.hidden, self.eps, _ptr(self.conv_weight),
                                    self.conv_kernel, self.conv_dilation)
            object.__setattr__(self, "_desc", d)
            object.__setattr__(self, "_desc_parts", (hd, td))
            object.__setattr__(self, "_ws_bytes", {})
        return d


def _batch(input_ids, query_start_loc, ngram_context=None, ngram_context_out=None, conv_state=None,
           conv_state_out=None, num_tokens=None, max_request_tokens=0, context_len=None,
           state_shape=None) -> capi.ple_batch_desc:
    """The batch descriptor, after checking its tensors: input_ids int32 [T],
    query_start_loc int32 [R+1], contexts int32 [R][context_len], conv states
    bf16 state_shape = (S, N) per request."""
    if input_ids is not None:
        _req("input_ids", input_ids, (None,), _I32)
    _req("query_start_loc", query_start_loc, (None,), _I32)
    T = int(input_ids.shape[0]) if input_ids is not None else int(num_tokens)
    R = int(query_start_loc.shape[0]) - 1
    if R < 0:
        raise ValueError("query_start_loc needs at least one entry")
    for name, c in (("ngram_context", ngram_context), ("ngram_context_out", ngram_context_out)):
        if c is not None:
            if context_len is None:
                raise ValueError(f"{name} given without the hash's context length")
            _req(name, c, (R, context_len), _I32)
    for name, c in (("conv_state", conv_state), ("conv_state_out", conv_state_out)):
        if c is not None:
            if state_shape is None:
                raise ValueError(f"{name} given without the conv shape")
            _req(name, c, (R, *state_shape), _BF16)
    _same_device(input_ids, query_start_loc, ngram_context, ngram_context_out, conv_state, conv_state_out)
    return capi.ple_batch_desc(_ptr(input_ids), _ptr(query_start_loc), T, R, int(max_request_tokens),
                               _ptr(ngram_context), _ptr(ngram_context_out), _ptr(conv_state), _ptr(conv_state_out))


def ple_ngram_ids(hash: HashParams, input_ids, query_start_loc, *, ngram_context=None, ngram_context_out=None,
                  ids=None, stream=None):
    T = input_ids.shape[0]
    if ids is None:
        ids = torch.empty((T, hash.num_heads), dtype=torch.int32, device=input_ids.device)
    _req("ids", ids, (T, hash.num_heads), _I32)
    h = hash.desc()
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, context_len=hash.context_len)
    _same_device(input_ids, ids)
    capi.check(capi.load().ple_ngram_ids(ctypes.byref(h), ctypes.byref(b), _ptr(ids), _stream(stream)),
               "ple_ngram_ids")
    return ids


def ple_gather(table: Table, ids, *, rows=None, stream=None):
    _req("ids", ids, (None, None), _I32)
    T, H = ids.shape
    if rows is None:
        rows = torch.empty((T, H * table.dim), dtype=torch.bfloat16, device=ids.device)
    _req("rows", rows, (T, H * table.dim), _BF16)
    _same_device(ids, rows)
    t = table.desc()
    capi.check(capi.load().ple_gather(ctypes.byref(t), _ptr(ids), T, H, _ptr(rows), _stream(stream)), "ple_gather")
    return rows


def ple_lookup(hash: HashParams, table: Table, input_ids, query_start_loc, *, ngram_context=None,
               ngram_context_out=None, ids_out=None, rows=None, stream=None):
    _req("input_ids", input_ids, (None,), _I32)
    T = input_ids.shape[0]
    if rows is None:
        rows = torch.empty((T, hash.num_heads * table.dim), dtype=torch.bfloat16, device=input_ids.device)
    _req("rows", rows, (T, hash.num_heads * table.dim), _BF16)
    _req("ids_out", ids_out, (T, hash.num_heads), _I32, optional=True)
    h, t = hash.desc(), table.desc()
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, context_len=hash.context_len)
    _same_device(input_ids, rows, ids_out)
    capi.check(capi.load().ple_lookup(ctypes.byref(h), ctypes.byref(t), ctypes.byref(b), _ptr(ids_out), _ptr(rows),
                                      _stream(stream)), "ple_lookup")
    return rows


def ple_prefetch(layer: Layer, input_ids, query_start_loc, staging, *, ngram_context=None, ngram_context_out=None,
                 stream=None):
    _req("input_ids", input_ids, (None,), _I32)
    _req("staging", staging, (input_ids.shape[0], layer.hash.num_heads * layer.table.dim), _BF16)
    L = layer.desc()
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, context_len=layer.hash.context_len)
    _same_device(input_ids, staging)
    capi.check(capi.load().ple_prefetch(ctypes.byref(L), ctypes.byref(b), _ptr(staging), _stream(stream)),
               "ple_prefetch")
    return staging


def ple_prefetch_dedup_workspace_bytes(max_tokens: int, num_heads: int) -> int:
    return int(capi.load().ple_prefetch_dedup_workspace_bytes(max_tokens, num_heads))


def ple_prefetch_dedup(layer: Layer, input_ids, query_start_loc, staging, *, workspace=None, num_unique=None,
                       ngram_context=None, ngram_context_out=None, stream=None):
    """ple_prefetch reading each distinct table row once; num_unique (device int32 [1]) receives
    the number of distinct rows."""
    _req("input_ids", input_ids, (None,), _I32)
    T = input_ids.shape[0]
    _req("staging", staging, (T, layer.hash.num_heads * layer.table.dim), _BF16)
    _req("num_unique", num_unique, (1,), _I32, optional=True)
    need = ple_prefetch_dedup_workspace_bytes(T, layer.hash.num_heads)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=input_ids.device)
    _req_bytes("workspace", workspace, need)
    L = layer.desc()
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, context_len=layer.hash.context_len)
    _same_device(input_ids, staging, num_unique, workspace)
    capi.check(capi.load().ple_prefetch_dedup(ctypes.byref(L), ctypes.byref(b), _ptr(staging), _ptr(workspace),
                                              _nbytes(workspace), _ptr(num_unique), _stream(stream)),
               "ple_prefetch_dedup")
    return staging


def ple_prefetch_dedup_plan(layer: Layer, input_ids, query_start_loc, workspace, *, ngram_context=None,
                            ngram_context_out=None, stream=None):
    """The first half of ple_prefetch_dedup: IDs, distinct-ID set and list into workspace."""
    _req("input_ids", input_ids, (None,), _I32)
    T = input_ids.shape[0]
    _req_bytes("workspace", workspace, ple_prefetch_dedup_workspace_bytes(T, layer.hash.num_heads))
    L = layer.desc()
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, context_len=layer.hash.context_len)
    _same_device(input_ids, workspace)
    capi.check(capi.load().ple_prefetch_dedup_plan(ctypes.byref(L), ctypes.byref(b), _ptr(workspace),
                                                   _nbytes(workspace), _stream(stream)), "ple_prefetch_dedup_plan")
    return workspace


def ple_prefetch_dedup_fetch(layer: Layer, num_tokens: int, workspace, staging, *, num_unique=None, stream=None):
    """The second half of ple_prefetch_dedup: the listed rows into staging, then the repeats;
    workspace as the plan for num_tokens tokens left it."""
    T = int(num_tokens)
    _req("staging", staging, (T, layer.hash.num_heads * layer.table.dim), _BF16)
    _req("num_unique", num_unique, (1,), _I32, optional=True)
    _req_bytes("workspace", workspace, ple_prefetch_dedup_workspace_bytes(T, layer.hash.num_heads))
    L = layer.desc()
    _same_device(staging, num_unique, workspace)
    capi.check(capi.load().ple_prefetch_dedup_fetch(ctypes.byref(L), T, _ptr(workspace), _nbytes(workspace),
                                                    _ptr(staging), _ptr(num_unique), _stream(stream)),
               "ple_prefetch_dedup_fetch")
    return staging


def _nbytes(t) -> int:
    return t.numel() * t.element_size() if isinstance(t, torch.Tensor) else (1 << 62)


def ple_dp_gather_slot(token_counts, group_size: int, dp_rank: int) -> tuple[int, int]:
    """(slot, offset) of dp_rank's tokens in its group's padded, rank-major gathered buffer."""
    c = np.ascontiguousarray(token_counts, dtype=np.int64)
    slot, off = ctypes.c_int64(), ctypes.c_int64()
    capi.check(capi.load().ple_dp_gather_slot(c.ctypes.data, len(c), group_size, dp_rank, ctypes.byref(slot),
                                              ctypes.byref(off)), "ple_dp_gather_slot")
    return slot.value, off.value


def ple_head_shard(num_heads: int, tp_size: int, tp_rank: int, dp_size: int, dp_rank: int) -> tuple[int, int]:
    """(first_head, shard_heads) of the TP-major head shard of (tp_rank, dp_rank)."""
    f, n = ctypes.c_int32(), ctypes.c_int32()
    capi.check(capi.load().ple_head_shard(num_heads, tp_size, tp_rank, dp_size, dp_rank, ctypes.byref(f),
                                          ctypes.byref(n)), "ple_head_shard")
    return f.value, n.value


def ple_select_rows(gathered, rank: int, num_tokens: int, *, out=None, stream=None):
    """gathered bf16 [E][E*slot][W] -> out bf16 [num_tokens][E*W] (rank's token window, shards in order)."""
    _req("gathered", gathered, (None, None, None), _BF16)
    E, rows, W = gathered.shape
    if E < 1 or rows % E != 0:
        raise ValueError(f"gathered has {rows} rows per shard, not a multiple of its {E} shards")
    slot = rows // E
    if out is None:
        out = torch.empty((num_tokens, E * W), dtype=torch.bfloat16, device=gathered.device)
    _req("out", out, (num_tokens, E * W), _BF16)
    _same_device(gathered, out)
    capi.check(capi.load().ple_select_rows(_ptr(gathered), E, slot, rank, num_tokens, W, _ptr(out),
                                           _stream(stream)), "ple_select_rows")
    return out


def ple_kv_proj(x, w, *, kv=None, stream=None):
    _req("x", x, (None, None), _BF16)
    T, K = x.shape
    _req("w", w, (None, K), _BF16)
    O = w.shape[0]
    if kv is None:
        kv = torch.empty((T, O), dtype=torch.bfloat16, device=x.device)
    _req("kv", kv, (T, O), _BF16)
    _same_device(x, w, kv)
    capi.check(capi.load().ple_kv_proj(_ptr(x), _ptr(w), T, K, O, _ptr(kv), _stream(stream)), "ple_kv_proj")
    return kv


def ple_gate(hidden, kv, *, eps: float = 1e-6, out=None, gate=None, want_gate: bool = True, stream=None):
    _req("hidden", hidden, (None, None), _BF16)
    T, N = hidden.shape
    _req("kv", kv, (T, 2 * N), _BF16)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=hidden.device)
    if gate is None and want_gate:
        gate = torch.empty((T,), dtype=torch.float32, device=hidden.device)
    _req("out", out, (T, N), _BF16)
    _req("gate", gate, (T,), _F32, optional=True)
    _same_device(hidden, kv, out, gate)
    capi.check(capi.load().ple_gate(_ptr(hidden), _ptr(kv), T, N, eps, _ptr(out), _ptr(gate), _stream(stream)),
               "ple_gate")
    return out, gate


def ple_conv(x, query_start_loc, w, *, dilation: int, conv_state=None, conv_state_out=None, y=None, stream=None):
    _req("x", x, (None, None), _BF16)
    T, N = x.shape
    _req("w", w, (N, None), _BF16)
    S = (int(w.shape[1]) - 1) * int(dilation)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _req("y", y, (T, N), _BF16)
    b = _batch(None, query_start_loc, conv_state=conv_state, conv_state_out=conv_state_out, num_tokens=T,
               state_shape=(S, N))
    _same_device(x, w, y, query_start_loc)
    capi.check(capi.load().ple_conv(_ptr(x), ctypes.byref(b), _ptr(w), N, w.shape[1], dilation, _ptr(y),
                                    _stream(stream)), "ple_conv")
    return y


def ple_spec_commit(input_ids, query_start_loc, accepted, *, hash: HashParams = None, ngram_context=None,
                    ngram_context_out=None, x=None, conv_kernel: int = 1, conv_dilation: int = 1, conv_state=None,
                    conv_state_out=None, stream=None):
    """State after a speculative verify step that keeps accepted[r] tokens of request r."""
    if x is not None:
        _req("x", x, (None, None), _BF16)
    N = int(x.shape[1]) if x is not None else (int(conv_state_out.shape[2]) if conv_state_out is not None else 0)
    S = (int(conv_kernel) - 1) * int(conv_dilation)
    R = int(query_start_loc.shape[0]) - 1
    _req("accepted", accepted, (R,), _I32)
    T = int(input_ids.shape[0]) if input_ids is not None else (x.shape[0] if x is not None else 0)
    if x is not None:
        _req("x", x, (T, N), _BF16)
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, conv_state, conv_state_out,
               num_tokens=None if input_ids is not None else T,
               context_len=hash.context_len if hash is not None else None, state_shape=(S, N))
    _same_device(input_ids, query_start_loc, accepted, x)
    h = hash.desc() if hash is not None else None
    capi.check(capi.load().ple_spec_commit(ctypes.byref(h) if h is not None else None, ctypes.byref(b),
                                           _ptr(accepted), _ptr(x), N, conv_kernel, conv_dilation, _stream(stream)),
               "ple_spec_commit")


def ple_prefill_workspace_bytes(layer: Layer, max_tokens: int) -> int:
    L = layer.desc()
    cache = layer._ws_bytes
    n = cache.get(max_tokens)
    if n is None:
        n = cache[max_tokens] = int(capi.load().ple_prefill_workspace_bytes(ctypes.byref(L), int(max_tokens)))
    return n


def prefill_conv_input(layer: Layer, workspace, num_tokens: int):
    """View of the conv input region (gated values, bf16 [T][N]) a ple_prefill_fused call leaves in its
    workspace: rows of each request's last S tokens and of requests of at most max(S, 16) tokens are
    set (every row after the decode tail)."""
    def r256(n):
        return (n + 255) // 256 * 256
    T, N = int(num_tokens), layer.hidden
    off = r256(T * layer.hash.num_heads * layer.table.dim * 2) + r256(T * 2 * N * 2)
    return workspace[off:off + T * N * 2].view(torch.bfloat16).view(T, N)


def prefill_kv(layer: Layer, workspace, num_tokens: int):
    """View of kv_proj's output (bf16 [T][2N]: key, then value) a ple_prefill_fused call leaves in its
    workspace."""
    def r256(n):
        return (n + 255) // 256 * 256
    T, N = int(num_tokens), layer.hidden
    off = r256(T * layer.hash.num_heads * layer.table.dim * 2)
    return workspace[off:off + T * 2 * N * 2].view(torch.bfloat16).view(T, 2 * N)


def ple_prefill_fused(layer: Layer, input_ids, query_start_loc, hidden, *, prefetched_rows=None, ngram_context=None,
                      ngram_context_out=None, conv_state=None, conv_state_out=None, out=None, gate=None,
                      workspace=None, max_request_tokens=0, stream=None):
    """max_request_tokens: 0 (unknown) or 1..4 (no request has more tokens: a decode step or
    speculative verify windows, run with one kernel for gate, conv and the carried state and
    context)."""
    _req("hidden", hidden, (None, layer.hidden), _BF16)
    T, N = hidden.shape
    _req("input_ids", input_ids, (T,), _I32)
    _req("prefetched_rows", prefetched_rows, (T, layer.hash.num_heads * layer.table.dim), _BF16, optional=True)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=hidden.device)
    _req("out", out, (T, N), _BF16)
    _req("gate", gate, (T,), _F32, optional=True)
    need = ple_prefill_workspace_bytes(layer, T)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=hidden.device)
    _req_bytes("workspace", workspace, need)
    L = layer.desc()
    S = (layer.conv_kernel - 1) * layer.conv_dilation
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, conv_state, conv_state_out,
               max_request_tokens=max_request_tokens, context_len=layer.hash.context_len, state_shape=(S, N))
    _same_device(input_ids, hidden, prefetched_rows, out, gate, workspace, layer.kv_weight, layer.conv_weight)
    capi.check(capi.load().ple_prefill_fused(ctypes.byref(L), ctypes.byref(b), _ptr(hidden), _ptr(prefetched_rows),
                                             _ptr(out), _ptr(gate), _ptr(workspace), _nbytes(workspace),
                                             _stream(stream)), "ple_prefill_fused")
    return out


def ple_prefill_fused_noalloc(layer: Layer, input_ids, query_start_loc, hidden, *, prefetched_rows=None,
                              ngram_context=None, ngram_context_out=None, conv_state=None, conv_state_out=None,
                              out, gate=None, max_request_tokens=0, stream=None):
    """ple_prefill_fused with its intermediates in the library's own scratch array (no workspace,
    no allocation by the library; `out` is the caller's)."""
    _req("hidden", hidden, (None, layer.hidden), _BF16)
    T, N = hidden.shape
    _req("input_ids", input_ids, (T,), _I32)
    _req("prefetched_rows", prefetched_rows, (T, layer.hash.num_heads * layer.table.dim), _BF16, optional=True)
    _req("out", out, (T, N), _BF16)
    _req("gate", gate, (T,), _F32, optional=True)
    L = layer.desc()
    S = (layer.conv_kernel - 1) * layer.conv_dilation
    b = _batch(input_ids, query_start_loc, ngram_context, ngram_context_out, conv_state, conv_state_out,
               max_request_tokens=max_request_tokens, context_len=layer.hash.context_len, state_shape=(S, N))
    _same_device(input_ids, hidden, prefetched_rows, out, gate, layer.kv_weight, layer.conv_weight)
    capi.check(capi.load().ple_prefill_fused_noalloc(ctypes.byref(L), ctypes.byref(b), _ptr(hidden),
                                                     _ptr(prefetched_rows), _ptr(out), _ptr(gate), _stream(stream)),
               "ple_prefill_fused_noalloc")
    return out


class HostBuffer:
    """Mapped pinned host memory from ple_host_alloc (freed by close() or at collection)."""

    def __init__(self, nbytes: int):
        h, d = ctypes.c_void_p(), ctypes.c_void_p()
        capi.check(capi.load().ple_host_alloc(int(nbytes), ctypes.byref(h), ctypes.byref(d)), "ple_host_alloc")
        self.host, self.device, self.nbytes = h.value, d.value, int(nbytes)

    def numpy(self, dtype, shape) -> np.ndarray:
        """A numpy view of the host side (valid while this object lives)."""
        buf = (ctypes.c_char * self.nbytes).from_address(self.host)
        return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(shape)

    def close(self):
        if self.host:
            capi.check(capi.load().ple_host_free(self.host), "ple_host_free")
            self.host = self.device = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ple_host_alloc(nbytes: int) -> HostBuffer:
    return HostBuffer(nbytes)


def ple_host_free(buf: HostBuffer) -> None:
    buf.close()


def ple_stream_create_cu_masked(num_cus: int) -> torch.cuda.ExternalStream:
    s = ctypes.c_void_p()
    capi.check(capi.load().ple_stream_create_cu_masked(int(num_cus), ctypes.byref(s)), "ple_stream_create_cu_masked")
    return torch.cuda.ExternalStream(s.value)


def ple_stream_destroy(stream) -> None:
    capi.check(capi.load().ple_stream_destroy(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream),
               "ple_stream_destroy")


def ple_error_message() -> str:
    return capi.error_message()


def ple_version() -> str:
    return capi.load().ple_version().decode()
