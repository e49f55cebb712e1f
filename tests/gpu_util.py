"""Helpers shared by the GPU parity tests (device transfers, bf16 comparisons)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as wl

DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_bf16(a_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between bf16 bit patterns (signed zeros equal)."""
    def key(x):
        u = np.asarray(x, dtype=np.int64)
        return np.where(u & 0x8000, 0x8000 - u, u)
    return np.abs(key(a) - key(b))


def hash_params(batch: wl.Batch, layer: int = 0, first_head: int = 0, num_heads: int | None = None):
    import layer_embedding_lookup_amd as ple
    cfg = batch.cfg
    H = cfg.H if num_heads is None else num_heads
    sl = slice(first_head, first_head + H)
    return ple.HashParams(batch.multipliers[layer][sl], batch.vocab_sizes[sl], batch.offsets[sl],
                          heads_per_ngram=cfg.heads_per_ngram, context_len=cfg.context_len, eos_token_id=wl.EOS,
                          first_head=first_head)


def oracle_ids(batch: wl.Batch, layer: int = 0, first_head: int = 0, num_heads: int | None = None,
               want_context_out: bool = False):
    import oracle
    cfg = batch.cfg
    H = cfg.H if num_heads is None else num_heads
    sl = slice(first_head, first_head + H)
    return oracle.ngram_ids(batch.input_ids, batch.qsl, batch.multipliers[layer][sl], batch.vocab_sizes[sl],
                            batch.offsets[sl], context_len=cfg.context_len, heads_per_ngram=cfg.heads_per_ngram,
                            eos_token_id=wl.EOS, ngram_context=batch.ngram_context, first_head=first_head,
                            num_heads=H, want_context_out=want_context_out)


def oracle_threads() -> int:
    """Worker threads for the oracle's per-token work: the host's CPU share, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_kv_proj_threaded(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """oracle.kv_proj on blocks of rows in parallel threads.  Each output row is
    the oracle's own computation on that row (the C call releases the GIL); the
    split only spreads independent rows over the host cores."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    T = x.shape[0]
    out = np.empty((T, w.shape[0]), dtype=np.uint16)
    if T == 0:
        return out
    n = oracle_threads()
    bounds = np.linspace(0, T, min(T, n) + 1).astype(np.int64)  # one block per thread: each call widens W once

    def one(i):
        lo, hi = int(bounds[i]), int(bounds[i + 1])
        if hi > lo:
            out[lo:hi] = oracle.kv_proj(np.ascontiguousarray(x[lo:hi]), w)

    with ThreadPoolExecutor(n) as ex:
        list(ex.map(one, range(len(bounds) - 1)))
    return out


GATE_REL_TOL = 1e-5
BF16_ABS_TOL = 2e-2


def last_rows_of_requests(qsl, S: int, T: int, window: int = 16) -> np.ndarray:
    """Boolean mask of the conv inputs the fused prefill leaves in its workspace: the tokens among
    the last S of their request, and every token of a request of at most `window` tokens."""
    q = np.asarray(qsl, dtype=np.int64)
    m = np.zeros(T, dtype=bool)
    for r in range(len(q) - 1):
        a, b = int(q[r]), int(q[r + 1])
        m[a if b - a <= window else max(a, b - S):b] = True
    return m


def _ulp_bits(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of one ulp of each bf16 value (2^(exponent - 7); the smallest normal's
    ulp for zeros and subnormals)."""
    e = (np.asarray(bits, dtype=np.uint16) >> 7) & 0xFF
    e = np.maximum(e, 1).astype(np.int64) - 7
    return np.where(e >= 1, e << 7, 1 << (6 + e)).astype(np.uint16)


def check_gate_conv_stages(hidden, kv_gpu, gate_gpu, gated_gpu, y_gpu, qsl, conv_w, dilation, eps, *,
                           conv_state=None, state_out_gpu=None, tokens=None, gated_rows=None):
    """Stage-wise parity of the gate and the conv: each compared with the oracle
    run on the GPU's own input to that stage (its kv, its conv input), so the
    fp32 gate is held to rel 1e-5 and the bf16 outputs to one ulp and max-abs
    2e-2, and the carried conv state is a bit-exact copy.  `tokens` restricts
    the comparison to those tokens (every token when None).  `gated_rows`
    (a token mask) says which rows of gated_gpu the GPU wrote; when it is
    given the conv is checked on the oracle's conv input from the GPU's kv,
    whose rows may differ from the GPU's own by one ulp."""
    import oracle
    T = hidden.shape[0]
    if T == 0:
        return
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    want_gated_all, g_want_all = oracle.gate(hidden, kv_gpu, eps)
    if gate_gpu is not None:
        np.testing.assert_allclose(np.asarray(gate_gpu, np.float64)[sel], g_want_all[sel], rtol=GATE_REL_TOL, atol=0)
    rows = np.ones(T, dtype=bool) if gated_rows is None else np.asarray(gated_rows, dtype=bool)
    chk = np.zeros(T, dtype=bool)
    chk[sel] = True
    chk &= rows
    if chk.any():
        assert np.abs(bf16_f64(gated_gpu[chk]) - bf16_f64(want_gated_all[chk])).max() <= BF16_ABS_TOL
        assert bf16_ulp_distance(gated_gpu[chk], want_gated_all[chk]).max() <= 1
    x_in = gated_gpu if gated_rows is None else want_gated_all
    y_want, st_want = oracle.conv(x_in, qsl, conv_w, dilation, state=conv_state, want_state_out=True)
    assert np.abs(bf16_f64(y_gpu[sel]) - bf16_f64(y_want[sel])).max() <= BF16_ABS_TOL
    # fp32 sum of Kc exact bf16 products: |error| <= gamma_Kc * sum |w x|, plus one bf16 ulp of the
    # result (both sides round to bf16); away from cancellation that is one ulp.  On the oracle's
    # conv input (inputs within one ulp of the GPU's) add sum |w| ulp(x).
    Kc = conv_w.shape[1]
    gamma = Kc * 2.0 ** -24 / (1 - Kc * 2.0 ** -24)
    absw = conv_w & np.uint16(0x7FFF)
    abst = None if conv_state is None else conv_state & np.uint16(0x7FFF)
    mag = bf16_f64(oracle.conv(x_in & np.uint16(0x7FFF), qsl, absw, dilation, state=abst)[sel])
    bound = gamma * mag * 1.01
    if gated_rows is not None:
        # a bf16 result per term can lose to rounding: bound sum |w| ulp(x) from above by 1.01 x its bf16
        bound = bound + 1.01 * bf16_f64(oracle.conv(_ulp_bits(x_in), qsl, absw, dilation,
                                                     state=None if conv_state is None else
                                                     np.zeros_like(conv_state))[sel])
    e = bf16_f64(y_want[sel])
    ulp = np.maximum(np.abs(e), 2.0 ** -126) * 2.0 ** -7
    assert (np.abs(bf16_f64(y_gpu[sel]) - e) <= bound + ulp).all()
    if gated_rows is None:
        d = bf16_ulp_distance(y_gpu[sel], y_want[sel])
        assert d[np.abs(e) > 1e-2].max(initial=0) <= 1
    if state_out_gpu is not None:
        if gated_rows is None:
            np.testing.assert_array_equal(state_out_gpu, st_want)
        else:
            assert bf16_ulp_distance(state_out_gpu, st_want).max() <= 1
