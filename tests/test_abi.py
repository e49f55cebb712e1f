"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

from layer_embedding_lookup_amd import capi

# These calls pass a fake device address and rely on host-side validation
# rejecting them first; they only run where no GPU could execute a launch.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-pointer validation tests run only on hosts without a GPU")

lib = capi.load()
E_ARG, E_UNSUP, E_WS = capi.PLE_ERR_INVALID_ARGUMENT, capi.PLE_ERR_UNSUPPORTED, capi.PLE_ERR_WORKSPACE

FAKE = 1 << 40  # a 256-aligned address that is never dereferenced: every call below fails validation first


def test_exports_every_header_function():
    names = capi.header_functions()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(capi._PROTOS)


def test_version_and_empty_message():
    assert b"gfx950" in lib.ple_version()
    assert isinstance(lib.ple_error_message(), bytes)


def _hash(H=4, hpn=2, C=2, first=0, V=None, off=None):
    V = np.asarray(V if V is not None else [101, 103, 107, 109][:H], np.int64)
    off = np.asarray(off if off is not None else np.concatenate([[0], np.cumsum(V)[:-1]]), np.int64)
    m = np.ones((max(H, 1), C + 1), np.int64)
    keep = (V, off, m)
    return capi.ple_hash_desc(H, hpn, C, first, 0, 0, m.ctypes.data, V.ctypes.data, off.ctypes.data), keep


def _table(rows=420, dim=32, dtype=capi.PLE_DTYPE_BF16, ptr=FAKE, scales=None, block_scales=None):
    return capi.ple_table_desc(ptr, rows, dim, dtype, scales, block_scales)


def _batch(T=8, R=2, ctx=None, ctx_out=None, state=None, state_out=None):
    return capi.ple_batch_desc(FAKE, FAKE, T, R, 0, ctx, ctx_out, state, state_out)


def _msg():
    return lib.ple_error_message().decode()


def test_ngram_ids_rejects():
    b = _batch()
    h, keep = _hash(H=0)
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(b), FAKE, None) == E_ARG
    assert "empty head shard" in _msg()
    h, keep = _hash(H=4, hpn=1, C=2)  # only 2 heads exist
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(b), FAKE, None) == E_ARG
    h, keep = _hash(C=8)
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(b), FAKE, None) == E_ARG
    h, keep = _hash(V=[101, 0, 107, 109])
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(b), FAKE, None) == E_ARG
    h, keep = _hash(V=[2 ** 31, 1, 1, 1])
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(b), FAKE, None) == E_ARG
    h, keep = _hash(off=[0, 2 ** 31 - 50, 0, 0])
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(b), FAKE, None) == E_UNSUP
    h, keep = _hash()
    assert lib.ple_ngram_ids(ctypes.byref(h), None, FAKE, None) == E_ARG
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(_batch(T=5, R=0)), FAKE, None) == E_ARG
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(_batch()), None, None) == E_ARG
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(_batch(ctx=FAKE, ctx_out=FAKE)), FAKE, None) == E_ARG
    assert "alias" in _msg()


def test_empty_batch_is_noop_without_device():
    h, keep = _hash()
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(_batch(T=0, R=0)), None, None) == capi.PLE_OK
    assert lib.ple_ngram_ids(ctypes.byref(h), ctypes.byref(_batch(T=0, R=3)), None, None) == capi.PLE_OK
    t = _table()
    assert lib.ple_lookup(ctypes.byref(h), ctypes.byref(t), ctypes.byref(_batch(T=0, R=0)), None, None,
                          None) == capi.PLE_OK
    assert lib.ple_gather(ctypes.byref(t), None, 0, 4, None, None) == capi.PLE_OK
    assert lib.ple_kv_proj(FAKE, FAKE, 0, 128, 256, FAKE, None) == capi.PLE_OK
    assert lib.ple_gate(FAKE, FAKE, 0, 128, 1e-6, FAKE, None, None) == capi.PLE_OK


def test_table_rejects():
    h, keep = _hash()
    b = _batch()
    for t, code in [(_table(dtype=7), E_UNSUP), (_table(ptr=None), E_ARG), (_table(ptr=FAKE + 8), E_ARG),
                    (_table(dim=12), E_UNSUP), (_table(dim=24, dtype=capi.PLE_DTYPE_FP8_E4M3, scales=FAKE), E_UNSUP),
                    (_table(dtype=capi.PLE_DTYPE_FP8_E4M3, scales=None), E_ARG), (_table(rows=0), E_ARG),
                    (_table(rows=300), E_ARG)]:  # rows 300 < 420 covered by the heads
        assert lib.ple_lookup(ctypes.byref(h), ctypes.byref(t), ctypes.byref(b), None, FAKE, None) == code, _msg()
    assert lib.ple_gather(ctypes.byref(_table()), FAKE, 4, 0, FAKE, None) == E_ARG
    assert lib.ple_gather(ctypes.byref(_table()), FAKE, 4, 33, FAKE, None) == E_ARG
    assert lib.ple_gather(ctypes.byref(_table()), FAKE, 4, 4, FAKE + 4, None) == E_ARG


def test_kv_proj_gate_conv_reject():
    assert lib.ple_kv_proj(FAKE, FAKE, 10, 100, 256, FAKE, None) == E_UNSUP
    assert lib.ple_kv_proj(FAKE, FAKE, 10, 128, 250, FAKE, None) == E_UNSUP
    assert lib.ple_kv_proj(FAKE, FAKE, 10, (1 << 20) + 64, 256, FAKE, None) == E_UNSUP
    assert lib.ple_kv_proj(None, FAKE, 10, 128, 256, FAKE, None) == E_ARG
    assert lib.ple_kv_proj(FAKE + 2, FAKE, 10, 128, 256, FAKE, None) == E_ARG
    assert lib.ple_kv_proj(FAKE, FAKE, -1, 128, 256, FAKE, None) == E_ARG
    assert lib.ple_gate(FAKE, FAKE, 4, 12, 1e-6, FAKE, None, None) == E_UNSUP
    assert lib.ple_gate(FAKE, FAKE, 4, 16, -1.0, FAKE, None, None) == E_ARG
    assert lib.ple_gate(FAKE, FAKE, 4, 16, float("nan"), FAKE, None, None) == E_ARG
    assert lib.ple_gate(FAKE, None, 4, 16, 1e-6, FAKE, None, None) == E_ARG
    b = _batch()
    assert lib.ple_conv(FAKE, ctypes.byref(b), FAKE, 16, 0, 1, FAKE + 256, None) == E_ARG
    assert lib.ple_conv(FAKE, ctypes.byref(b), FAKE, 16, 4, 0, FAKE + 256, None) == E_ARG
    assert lib.ple_conv(FAKE, ctypes.byref(b), FAKE, 16, 17, 1, FAKE + 256, None) == E_ARG
    assert lib.ple_conv(FAKE, ctypes.byref(b), FAKE, 12, 4, 1, FAKE + 256, None) == E_UNSUP
    assert lib.ple_conv(FAKE, ctypes.byref(b), FAKE, 16, 4, 1, FAKE, None) == E_ARG  # y aliases x
    bs = _batch(state=FAKE, state_out=FAKE)
    assert lib.ple_conv(FAKE, ctypes.byref(bs), FAKE, 16, 4, 1, FAKE + 256, None) == E_ARG
    assert "alias" in _msg()


def _layer(N=128, Kc=4, d=2, kvw=FAKE, convw=FAKE, eps=1e-6):
    h, keep = _hash()
    return capi.ple_layer_desc(h, _table(), kvw, N, eps, convw, Kc, d), keep


def test_prefill_workspace():
    L, keep = _layer()
    need = lib.ple_prefill_workspace_bytes(ctypes.byref(L), 24)
    # rows 24 x 128 bf16, kv 24 x 256 bf16, conv input 24 x 128 bf16, gate 24 fp32, each rounded up
    # to 256 bytes
    assert need == 6144 + 12288 + 6144 + 256
    b = _batch(T=24, R=4)
    rc = lib.ple_prefill_fused(ctypes.byref(L), ctypes.byref(b), FAKE, None, FAKE, None, FAKE, need - 1, None)
    assert rc == E_WS
    rc = lib.ple_prefill_fused(ctypes.byref(L), ctypes.byref(b), FAKE, None, FAKE, None, FAKE + 16, need, None)
    assert rc == E_WS
    rc = lib.ple_prefill_fused(ctypes.byref(L), ctypes.byref(b), FAKE, None, FAKE, None, None, need, None)
    assert rc == E_WS
    L2, keep2 = _layer(N=100)
    assert lib.ple_prefill_fused(ctypes.byref(L2), ctypes.byref(b), FAKE, None, FAKE, None, FAKE, need,
                                 None) == E_UNSUP
    L3, keep3 = _layer(eps=-1.0)
    assert lib.ple_prefill_fused(ctypes.byref(L3), ctypes.byref(b), FAKE, None, FAKE, None, FAKE, need, None) == E_ARG
    assert lib.ple_prefill_fused(None, ctypes.byref(b), FAKE, None, FAKE, None, FAKE, need, None) == E_ARG


def test_host_and_stream_args():
    h = ctypes.c_void_p()
    d = ctypes.c_void_p()
    assert lib.ple_host_alloc(0, ctypes.byref(h), ctypes.byref(d)) == E_ARG
    assert lib.ple_host_free(None) == capi.PLE_OK
    s = ctypes.c_void_p()
    assert lib.ple_stream_create_cu_masked(0, ctypes.byref(s)) == E_ARG
    assert lib.ple_stream_destroy(None) == capi.PLE_OK


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(capi, "_lib", None)
    monkeypatch.setattr(capi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        capi.load()


def test_table_formats_rejected_before_any_launch():
    h, keep = _hash()
    b = _batch()
    for t, code, text in [
            (_table(dtype=capi.PLE_DTYPE_FP8_E4M3_GLOBAL), E_ARG, "row_scales"),
            (_table(dtype=capi.PLE_DTYPE_NVFP4, scales=FAKE), E_ARG, "block_scales"),
            (_table(dtype=capi.PLE_DTYPE_NVFP4, dim=48, scales=FAKE, block_scales=FAKE), E_UNSUP, "16 bytes"),
            (_table(dtype=capi.PLE_DTYPE_NVFP4, scales=FAKE, block_scales=FAKE + 1), E_ARG, "2-byte"),
            (_table(dtype=7), E_UNSUP, "PLE_DTYPE")]:
        assert lib.ple_lookup(ctypes.byref(h), ctypes.byref(t), ctypes.byref(b), None, FAKE, None) == code
        assert text in _msg()


def test_dedup_workspace_size_and_limits():
    f = lib.ple_prefetch_dedup_workspace_bytes
    # T*H = 24*4 = 96 rows: IDs, slots, list of distinct rows and list of repeats 96*4 bytes each
    # (256-rounded), the lists' counts (256), hash set of 256 slots x 2 (keys, first position)
    assert f(24, 4) == 4 * 512 + 256 + 2 * 1024
    assert f(8192, 8) == 4 * 65536 * 4 + 256 + 2 * 131072 * 4
    assert f(0, 8) == 0 and f(1 << 22, 2) == 0  # beyond 2^22 rows: unsupported
    h, keep = _hash()
    layer = capi.ple_layer_desc(h, _table(), FAKE, 128, 1e-6, FAKE, 4, 2)
    b = _batch()
    assert lib.ple_prefetch_dedup(ctypes.byref(layer), ctypes.byref(b), FAKE, FAKE, 16, None, None) == E_WS
    assert lib.ple_prefetch_dedup(ctypes.byref(layer), ctypes.byref(b), FAKE, FAKE + 4, 1 << 20, None, None) == E_WS
    big = capi.ple_batch_desc(FAKE, FAKE, 1 << 21, 2, 0, None, None, None, None)
    assert lib.ple_prefetch_dedup(ctypes.byref(layer), ctypes.byref(big), FAKE, FAKE, 1 << 30, None, None) == E_UNSUP
    assert lib.ple_prefetch_dedup(None, ctypes.byref(b), FAKE, FAKE, 1 << 20, None, None) == E_ARG
    # the two halves check the same things before any device call
    assert lib.ple_prefetch_dedup_plan(ctypes.byref(layer), ctypes.byref(b), FAKE, 16, None) == E_WS
    assert lib.ple_prefetch_dedup_plan(ctypes.byref(layer), ctypes.byref(big), FAKE, 1 << 30, None) == E_UNSUP
    assert lib.ple_prefetch_dedup_plan(None, ctypes.byref(b), FAKE, 1 << 20, None) == E_ARG
    assert lib.ple_prefetch_dedup_plan(ctypes.byref(layer), None, FAKE, 1 << 20, None) == E_ARG
    assert lib.ple_prefetch_dedup_fetch(ctypes.byref(layer), b.num_tokens, FAKE + 4, 1 << 20, FAKE, None, None) == E_WS
    assert lib.ple_prefetch_dedup_fetch(ctypes.byref(layer), b.num_tokens, FAKE, 1 << 20, FAKE + 2, None, None) == E_ARG
    assert lib.ple_prefetch_dedup_fetch(ctypes.byref(layer), -1, FAKE, 1 << 20, FAKE, None, None) == E_ARG
    assert lib.ple_prefetch_dedup_fetch(ctypes.byref(layer), 1 << 21, FAKE, 1 << 30, FAKE, None, None) == E_UNSUP
    assert lib.ple_prefetch_dedup_fetch(None, b.num_tokens, FAKE, 1 << 20, FAKE, None, None) == E_ARG
    # nothing to do: no device call
    assert lib.ple_prefetch_dedup_fetch(ctypes.byref(layer), 0, None, 0, None, None, None) == 0


def test_spec_commit_rejects_and_noops():
    h, keep = _hash()
    acc = FAKE + 512
    # Nothing to write: returns before any device call.
    assert lib.ple_spec_commit(ctypes.byref(h), ctypes.byref(_batch()), acc, FAKE, 16, 4, 1, None) == capi.PLE_OK
    assert lib.ple_spec_commit(ctypes.byref(h), ctypes.byref(_batch(T=0, R=0, ctx_out=FAKE, state_out=FAKE)), None,
                               None, 16, 4, 1, None) == capi.PLE_OK
    assert lib.ple_spec_commit(ctypes.byref(h), None, acc, FAKE, 16, 4, 1, None) == E_ARG
    # Context output needs the hash (C, EOS); conv state output needs a valid conv shape and x.
    assert lib.ple_spec_commit(None, ctypes.byref(_batch(ctx_out=FAKE)), acc, None, 0, 1, 1, None) == E_ARG
    bs = _batch(state_out=FAKE)
    assert lib.ple_spec_commit(None, ctypes.byref(bs), acc, FAKE, 12, 4, 1, None) == E_UNSUP
    assert lib.ple_spec_commit(None, ctypes.byref(bs), acc, FAKE, 16, 17, 1, None) == E_ARG
    assert lib.ple_spec_commit(None, ctypes.byref(bs), acc, FAKE, 16, 4, 0, None) == E_ARG
    assert lib.ple_spec_commit(None, ctypes.byref(bs), acc, None, 16, 4, 1, None) == E_ARG
    assert lib.ple_spec_commit(None, ctypes.byref(bs), acc, FAKE + 2, 16, 4, 1, None) == E_ARG
    assert lib.ple_spec_commit(None, ctypes.byref(bs), None, FAKE, 16, 4, 1, None) == E_ARG
    assert "accepted" in _msg()
    assert lib.ple_spec_commit(None, ctypes.byref(bs), acc + 2, FAKE, 16, 4, 1, None) == E_ARG
    b_alias = _batch(state=FAKE + 256, state_out=FAKE + 256)
    assert lib.ple_spec_commit(None, ctypes.byref(b_alias), acc, FAKE, 16, 4, 1, None) == E_ARG
    assert "alias" in _msg()


def test_prefill_noalloc_rejects_beyond_its_scratch():
    """The allocation-free fused prefill takes at most PLE_NOALLOC_SCRATCH_BYTES of intermediates and
    says so before any device work; its argument checks are those of ple_prefill_fused."""
    L, keep = _layer()
    # 128-wide rows, kv and conv input: (128 + 256 + 128) * 2 bytes per token
    per_token = (128 + 256 + 128) * 2
    T = capi.PLE_NOALLOC_SCRATCH_BYTES // per_token + 1
    b = capi.ple_batch_desc(FAKE, FAKE, T, 4, 0, None, None, None, None)
    assert lib.ple_prefill_fused_noalloc(ctypes.byref(L), ctypes.byref(b), FAKE, None, FAKE + 256, None,
                                         None) == E_WS
    assert "scratch" in _msg()
    L3, keep3 = _layer(eps=-1.0)
    b = _batch(T=24, R=4)
    assert lib.ple_prefill_fused_noalloc(ctypes.byref(L3), ctypes.byref(b), FAKE, None, FAKE, None, None) == E_ARG
    assert lib.ple_prefill_fused_noalloc(None, ctypes.byref(b), FAKE, None, FAKE, None, None) == E_ARG
    L2, keep2 = _layer(N=100)
    assert lib.ple_prefill_fused_noalloc(ctypes.byref(L2), ctypes.byref(b), FAKE, None, FAKE, None, None) == E_UNSUP


def test_bench_library_exports_its_header():
    """libple_bench (the benchmark's streaming-copy ceilings) loads and exports what
    include/ple_bench.h declares; bad arguments are refused before any launch."""
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(root, "include", "ple_bench.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(ple_bench_[a-z_]+)\s*\(", text)))
    assert names == ["ple_bench_copy", "ple_bench_copy_rows", "ple_bench_error_message", "ple_bench_gather_expand"]
    blib = ctypes.CDLL(os.path.join(root, "layer_embedding_lookup_amd", "libple_bench.so"))
    for n in names:
        assert hasattr(blib, n)
    blib.ple_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    blib.ple_bench_copy_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert blib.ple_bench_copy(FAKE, FAKE + 256, 24, None) == E_ARG
    assert blib.ple_bench_copy(FAKE + 8, FAKE + 256, 32, None) == E_ARG
    assert blib.ple_bench_copy(FAKE, FAKE + 256, 0, None) == capi.PLE_OK
    assert blib.ple_bench_copy_rows(FAKE, 10, 24, FAKE, 4, FAKE, None) == E_ARG
    assert blib.ple_bench_copy_rows(FAKE, 10, 1024, FAKE, 0, FAKE, None) == capi.PLE_OK
    blib.ple_bench_gather_expand.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p]
    ge = blib.ple_bench_gather_expand
    assert ge(FAKE, 10, 3, None, 0, FAKE, 4, 1024, FAKE, None) == E_ARG       # expand 1, 2 or 4
    assert ge(FAKE, 10, 2, None, 1, FAKE, 4, 1024, FAKE, None) == E_ARG       # a side read needs aux
    assert ge(FAKE, 10, 2, FAKE + 2, 1, FAKE, 4, 1024, FAKE, None) == E_ARG   # word-aligned aux
    assert ge(FAKE, 10, 4, FAKE, 2, FAKE, 4, 1000, FAKE, None) == E_ARG       # power-of-two rows
    assert ge(FAKE, 10, 4, FAKE, 2, FAKE, 0, 1024, FAKE, None) == capi.PLE_OK
