"""Brute-force n-gram enumeration with Python big integers (tiny inputs only).

An independent second statement of the n-gram ID definition, used to pin the
oracle.  It differs from the oracle in form on purpose:
  * each request is materialised as the token sequence ``context ++ tokens``
    (context defaulting to EOS), and windows are slices of that sequence;
  * the EOS rule is applied by an explicit backward scan of each window;
  * the hash sum is exact (multipliers taken as signed 64-bit values), then
    brought to the signed 64-bit range by ((S + 2^63) mod 2^64) - 2^63, and
    reduced with Python's floor ``%``.
Source: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels", sections
实现拆解 (ids kernel: ragged requests, EOS replacement, int64 overflow) and
关键源码片段 (the per-shift loop over the preceding tokens).
"""
from __future__ import annotations

import numpy as np


def to_signed64(v: int) -> int:
    return ((v + (1 << 63)) % (1 << 64)) - (1 << 63)


def ngram_ids(tokens, qsl, mults, vocab, offsets, *, context_len, heads_per_ngram, eos,
              context=None, first_head=0):
    tokens = [int(x) for x in tokens]
    qsl = [int(x) for x in qsl]
    H = len(vocab)
    C = context_len
    out = [[None] * H for _ in tokens]
    ctx_out = []
    for r in range(len(qsl) - 1):
        a, b = qsl[r], qsl[r + 1]
        prefix = [eos] * C if context is None else [int(x) for x in context[r]]
        seq = prefix + tokens[a:b]
        ctx_out.append(seq[len(seq) - C:])
        for i in range(C, len(seq)):
            # window newest first: seq[i], seq[i-1], ..., seq[i-C]
            window = [seq[i - j] for j in range(C + 1)]
            masked = list(window)
            seen = False
            for j in range(1, C + 1):
                if window[j] == eos:
                    seen = True
                if seen:
                    masked[j] = eos
            for h in range(H):
                n = 2 + (first_head + h) // heads_per_ngram
                m = [int(x) for x in mults[h]]
                m = [x - (1 << 64) if x >= (1 << 63) else x for x in m]
                total = sum(masked[j] * m[j] for j in range(n))
                out[a + (i - C)][h] = offsets[h] + to_signed64(total) % vocab[h]
    return np.asarray(out, dtype=np.int64).reshape(len(tokens), H), np.asarray(ctx_out, dtype=np.int64)
