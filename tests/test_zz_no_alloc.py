"""The allocation-free fused prefill (ple_prefill_fused_noalloc) through the
C ABI: its intermediates live in the library's own scratch array, so three
calls in a row, each smaller than the one before (a 1536-token prefill with
carried context and conv state, a 256-request decode step on the one-kernel
decode tail, the tiny 4-request batch), must give the same bits as
ple_prefill_fused with a fresh workspace, whatever the earlier calls left in
the array; the tiny batch also against the oracle.  A batch whose
intermediates exceed the array is refused before any device work."""
import dataclasses

import numpy as np
import pytest
import torch

import layer_embedding_lookup_amd as ple
import oracle
import workloads as wl
from gpu_util import DEV, bf16_f64, dev, dev_bf16, hash_params, host_bits, log

pytestmark = pytest.mark.gpu


def _setup(cfg, hint):
    b = wl.make_batch(cfg, with_context=True, with_state=True)
    table, _ = wl.make_table(cfg)
    kvw, cw, hidden = wl.make_kv_weight(cfg), wl.make_conv_weight(cfg), wl.make_hidden(cfg)
    keep = dev_bf16(table)
    L = ple.Layer(hash_params(b), ple.Table.from_tensor(keep), dev_bf16(kvw), dev_bf16(cw),
                  conv_dilation=cfg.conv_dilation, eps=cfg.eps)
    args = dict(input_ids=dev(b.input_ids), query_start_loc=dev(b.qsl), hidden=dev_bf16(hidden),
                ngram_context=dev(b.ngram_context), conv_state=dev_bf16(b.conv_state))
    return dict(cfg=cfg, b=b, L=L, args=args, hint=hint, host=(table, kvw, cw, hidden), keep=keep)


def _outputs(case):
    cfg, b = case["cfg"], case["b"]
    return dict(out=torch.full((cfg.T, cfg.N), 3.0, dtype=torch.bfloat16, device=DEV),
                gate=torch.full((cfg.T,), -1.0, dtype=torch.float32, device=DEV),
                conv_state_out=torch.full((b.R, cfg.S, cfg.N), 5.0, dtype=torch.bfloat16, device=DEV),
                ngram_context_out=torch.full((b.R, cfg.context_len), -7, dtype=torch.int32, device=DEV))


def _host(o):
    return {k: (host_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in o.items()}


def test_noalloc_equals_workspace_path_three_calls_shrinking():
    cases = [
        _setup(dataclasses.replace(wl.CONFIGS[3], idx=71, T=1536, vocab_base=5003), 0),
        _setup(dataclasses.replace(wl.CONFIGS[2], idx=72, vocab_base=4001), 1),
        _setup(wl.CONFIGS[1], 0),
    ]
    refs = []
    for c in cases:
        o = _outputs(c)
        ple.ple_prefill_fused(c["L"], **c["args"], max_request_tokens=c["hint"], **o)
        refs.append(o)
    torch.cuda.synchronize()
    got = []
    for c in cases:  # the allocation-free calls back to back, each smaller than the last
        need = ple.ple_prefill_workspace_bytes(c["L"], c["cfg"].T)
        log(f"noalloc {c['cfg'].name}: T={c['cfg'].T}, {need} bytes of intermediates")
        assert need <= ple.capi.PLE_NOALLOC_SCRATCH_BYTES
        o = _outputs(c)
        ple.ple_prefill_fused_noalloc(c["L"], **c["args"], max_request_tokens=c["hint"], **o)
        got.append(o)
    torch.cuda.synchronize()
    for c, r, g in zip(cases, refs, got):
        hr, hg = _host(r), _host(g)
        for k in hr:
            np.testing.assert_array_equal(hg[k], hr[k], err_msg=f"{c['cfg'].name}: {k}")
    # the tiny batch against the oracle as well
    c, hg = cases[2], _host(got[2])
    cfg, b = c["cfg"], c["b"]
    table, kvw, cw, hidden = c["host"]
    ids_args = dict(input_ids=b.input_ids, qsl=b.qsl, multipliers=b.multipliers[0], vocab_sizes=b.vocab_sizes,
                    offsets=b.offsets, context_len=cfg.context_len, heads_per_ngram=cfg.heads_per_ngram,
                    eos_token_id=wl.EOS, ngram_context=b.ngram_context)
    ref = oracle.prefill(ids_args, table, None, hidden, kvw, cw, cfg.conv_dilation, qsl=b.qsl, eps=cfg.eps,
                         conv_state=b.conv_state)
    assert np.abs(bf16_f64(hg["out"]) - bf16_f64(ref["y"])).max() <= 2e-2


def test_noalloc_refuses_beyond_its_scratch():
    cfg = dataclasses.replace(wl.CONFIGS[3], idx=73, T=2100, vocab_base=5003)
    c = _setup(cfg, 0)
    assert ple.ple_prefill_workspace_bytes(c["L"], cfg.T) > ple.capi.PLE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(RuntimeError, match="scratch"):
        ple.ple_prefill_fused_noalloc(c["L"], **c["args"], out=torch.empty((cfg.T, cfg.N), dtype=torch.bfloat16,
                                                                             device=DEV))
