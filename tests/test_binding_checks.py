"""The Python binding checks every tensor behind a pointer (dtype, shape,
contiguity, device) on the host before it calls the library, so a mismatched
tensor raises instead of becoming an out-of-bounds device access.  These run
on the CPU: the library is replaced by a stub that fails the test if any call
reaches it (the workspace size queries, host arithmetic only, go through)."""
import numpy as np
import pytest
import torch

import layer_embedding_lookup_amd as ple
from layer_embedding_lookup_amd import capi


SIZE_QUERIES = ("ple_prefill_workspace_bytes", "ple_prefetch_dedup_workspace_bytes")


class _StubLibrary:
    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in SIZE_QUERIES:
            return getattr(self._real, name)
        raise AssertionError(f"the binding called {name} before rejecting the arguments")


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    stub = _StubLibrary(capi.load())
    monkeypatch.setattr(capi, "load", lambda: stub)


BF = torch.bfloat16


def _hash(H=4, C=2):
    return ple.HashParams(np.ones((H, C + 1), np.int64), [101, 103, 107, 109][:H], [0, 101, 204, 311][:H],
                          heads_per_ngram=H // C, context_len=C, eos_token_id=0)


def _table(D=32):
    return ple.Table(1 << 40, 420, D, ple.PLE_DTYPE_BF16)


def _layer(N=128, Kc=4, D=32):
    return ple.Layer(_hash(), _table(D), torch.zeros((2 * N, 4 * D), dtype=BF), torch.zeros((N, Kc), dtype=BF),
                     conv_dilation=2)


def test_kv_proj_shapes():
    x = torch.zeros((8, 128), dtype=BF)
    with pytest.raises(ValueError, match=r"w has shape \(256, 64\), expected \(\*, 128\)"):
        ple.ple_kv_proj(x, torch.zeros((256, 64), dtype=BF))
    with pytest.raises(ValueError, match=r"kv has shape \(8, 128\), expected \(8, 256\)"):
        ple.ple_kv_proj(x, torch.zeros((256, 128), dtype=BF), kv=torch.zeros((8, 128), dtype=BF))
    with pytest.raises(ValueError, match="dtype"):
        ple.ple_kv_proj(x.float(), torch.zeros((256, 128), dtype=BF))
    with pytest.raises(ValueError, match="contiguous"):
        ple.ple_kv_proj(torch.zeros((128, 8), dtype=BF).t(), torch.zeros((256, 128), dtype=BF))
    # right shapes, host tensors: rejected as not on a GPU, still before the library
    with pytest.raises(ValueError, match="GPU tensors"):
        ple.ple_kv_proj(x, torch.zeros((256, 128), dtype=BF))


def test_gate_shapes():
    h = torch.zeros((5, 16), dtype=BF)
    with pytest.raises(ValueError, match=r"kv has shape \(5, 16\), expected \(5, 32\)"):
        ple.ple_gate(h, torch.zeros((5, 16), dtype=BF))
    with pytest.raises(ValueError, match=r"gate has dtype"):
        ple.ple_gate(h, torch.zeros((5, 32), dtype=BF), gate=torch.zeros((5,), dtype=BF))
    with pytest.raises(ValueError, match=r"out has shape"):
        ple.ple_gate(h, torch.zeros((5, 32), dtype=BF), out=torch.zeros((4, 16), dtype=BF))


def test_conv_shapes():
    x = torch.zeros((10, 16), dtype=BF)
    qsl = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match=r"w has shape \(8, 4\), expected \(16, \*\)"):
        ple.ple_conv(x, qsl, torch.zeros((8, 4), dtype=BF), dilation=2)
    with pytest.raises(ValueError, match=r"conv_state has shape \(2, 5, 16\), expected \(2, 6, 16\)"):
        ple.ple_conv(x, qsl, torch.zeros((16, 4), dtype=BF), dilation=2, conv_state=torch.zeros((2, 5, 16), dtype=BF))
    with pytest.raises(ValueError, match=r"query_start_loc has dtype"):
        ple.ple_conv(x, qsl.long(), torch.zeros((16, 4), dtype=BF), dilation=2)


def test_lookup_and_ids_shapes():
    hp, tb = _hash(), _table()
    toks = torch.zeros((6,), dtype=torch.int32)
    qsl = torch.tensor([0, 6], dtype=torch.int32)
    with pytest.raises(ValueError, match=r"rows has shape \(6, 64\), expected \(6, 128\)"):
        ple.ple_lookup(hp, tb, toks, qsl, rows=torch.zeros((6, 64), dtype=BF))
    with pytest.raises(ValueError, match=r"ids_out has shape"):
        ple.ple_lookup(hp, tb, toks, qsl, rows=torch.zeros((6, 128), dtype=BF),
                       ids_out=torch.zeros((6, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match=r"ngram_context has shape \(1, 3\), expected \(1, 2\)"):
        ple.ple_ngram_ids(hp, toks, qsl, ngram_context=torch.zeros((1, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match=r"ids has shape"):
        ple.ple_ngram_ids(hp, toks, qsl, ids=torch.zeros((5, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match=r"input_ids has dtype"):
        ple.ple_ngram_ids(hp, toks.long(), qsl)
    with pytest.raises(ValueError, match=r"rows has shape"):
        ple.ple_gather(tb, torch.zeros((6, 4), dtype=torch.int32), rows=torch.zeros((6, 100), dtype=BF))


def test_layer_and_fused_shapes():
    with pytest.raises(ValueError, match=r"kv_weight has shape \(256, 64\), expected \(256, 128\)"):
        ple.Layer(_hash(), _table(), torch.zeros((256, 64), dtype=BF), torch.zeros((128, 4), dtype=BF),
                  conv_dilation=2)
    L = _layer()
    toks = torch.zeros((6,), dtype=torch.int32)
    qsl = torch.tensor([0, 6], dtype=torch.int32)
    with pytest.raises(ValueError, match=r"hidden has shape \(6, 64\), expected \(\*, 128\)"):
        ple.ple_prefill_fused(L, toks, qsl, torch.zeros((6, 64), dtype=BF))
    with pytest.raises(ValueError, match=r"input_ids has shape \(6,\), expected \(5,\)"):
        ple.ple_prefill_fused(L, toks, qsl, torch.zeros((5, 128), dtype=BF))
    with pytest.raises(ValueError, match=r"prefetched_rows has shape"):
        ple.ple_prefill_fused(L, toks, qsl, torch.zeros((6, 128), dtype=BF),
                              prefetched_rows=torch.zeros((6, 64), dtype=BF))
    with pytest.raises(ValueError, match=r"conv_state_out has shape \(1, 6, 64\), expected \(1, 6, 128\)"):
        ple.ple_prefill_fused(L, toks, qsl, torch.zeros((6, 128), dtype=BF),
                              conv_state_out=torch.zeros((1, 6, 64), dtype=BF))
    with pytest.raises(ValueError, match=r"workspace holds 16 bytes"):
        ple.ple_prefill_fused(L, toks, qsl, torch.zeros((6, 128), dtype=BF),
                              workspace=torch.zeros((16,), dtype=torch.uint8))


def test_spec_commit_and_select_shapes():
    qsl = torch.tensor([0, 2, 4], dtype=torch.int32)
    with pytest.raises(ValueError, match=r"accepted has shape \(3,\), expected \(2,\)"):
        ple.ple_spec_commit(torch.zeros((4,), dtype=torch.int32), qsl, torch.zeros((3,), dtype=torch.int32))
    with pytest.raises(ValueError, match=r"conv_state_out has shape"):
        ple.ple_spec_commit(torch.zeros((4,), dtype=torch.int32), qsl, torch.zeros((2,), dtype=torch.int32),
                            x=torch.zeros((4, 16), dtype=BF), conv_kernel=4, conv_dilation=1,
                            conv_state_out=torch.zeros((2, 2, 16), dtype=BF))
    with pytest.raises(ValueError, match=r"out has shape"):
        ple.ple_select_rows(torch.zeros((2, 8, 16), dtype=BF), 0, 3, out=torch.zeros((3, 16), dtype=BF))
    with pytest.raises(ValueError, match="multiple of its"):
        ple.ple_select_rows(torch.zeros((2, 7, 16), dtype=BF), 0, 3)
