"""Pins of the oracle's speculative-decode commit (``oracle.spec_commit``).

Source: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels", 实现拆解
items 4-5 (a speculative variant of the short conv; the short-conv backend
carries state between steps).  The pages fix no state layout; the reading is
that the state after a verify step equals the state of a run over the kept
tokens only.  The pins below do not reuse that construction:

* hand cases: the state rows and context tokens written out by hand;
* k single-token decode steps leave the same state as one commit of k tokens;
* accepting every token equals the plain state-out of the whole window;
* accepting none leaves the input state unchanged (NULL state -> zeros / EOS);
* counts outside 0..window length clamp.
"""
import numpy as np
import pytest

import oracle

EOS = 0


def _hash_args(C):
    H = C  # one head per order
    return dict(multipliers=np.ones((H, C + 1), np.int64) * 3, vocab_sizes=np.arange(101, 101 + 2 * H, 2),
                offsets=np.arange(H) * 1000, context_len=C, heads_per_ngram=1, eos_token_id=EOS)


def _rows(vals, N=8):
    """Rows of bf16 bit patterns, row i filled with vals[i]."""
    return np.repeat(np.asarray(vals, np.uint16)[:, None], N, axis=1)


@pytest.mark.parametrize("acc,want", [(0, [0x10, 0x11]), (1, [0x11, 0x20]), (2, [0x20, 0x21]), (4, [0x22, 0x23])])
def test_conv_state_hand_case(acc, want):
    # K=3, d=1 -> S=2; one request with a window of 4 tokens.
    x = _rows([0x20, 0x21, 0x22, 0x23])
    st = _rows([0x10, 0x11])[None]
    so, _ = oracle.spec_commit(None, x, [0, 4], [acc], conv_kernel=3, dilation=1, conv_state=st)
    np.testing.assert_array_equal(so[0], _rows(want))


def test_conv_state_hand_case_dilated_two_requests():
    # K=2, d=3 -> S=3.  Request 0 keeps 1 of 3 tokens, request 1 keeps 2 of 2.
    x = _rows([0x40, 0x41, 0x42, 0x50, 0x51])
    st = np.stack([_rows([1, 2, 3]), _rows([4, 5, 6])])
    so, _ = oracle.spec_commit(None, x, [0, 3, 5], [1, 2], conv_kernel=2, dilation=3, conv_state=st)
    np.testing.assert_array_equal(so[0], _rows([2, 3, 0x40]))
    np.testing.assert_array_equal(so[1], _rows([6, 0x50, 0x51]))


@pytest.mark.parametrize("acc,ctx,want", [(0, [5, 6], [5, 6]), (1, [5, 6], [6, 7]), (2, [5, 6], [7, 8]),
                                          (3, [5, 6], [8, 9]), (1, None, [EOS, 7]), (0, None, [EOS, EOS])])
def test_context_hand_case(acc, ctx, want):
    tok = np.asarray([7, 8, 9], np.int32)
    c = None if ctx is None else np.asarray([ctx], np.int32)
    _, co = oracle.spec_commit(tok, None, [0, 3], [acc], conv_kernel=1, dilation=1, hash_args=_hash_args(2),
                               ngram_context=c)
    assert co[0].tolist() == want


def test_counts_clamp():
    tok = np.asarray([7, 8, 9, 10], np.int32)
    x = _rows([1, 2, 3, 4])
    st = _rows([0x30, 0x31, 0x32])[None].repeat(2, axis=0)
    ctx = np.asarray([[5, 6], [15, 16]], np.int32)
    qsl = [0, 3, 4]
    hi = oracle.spec_commit(tok, x, qsl, [99, 1], conv_kernel=4, dilation=1, conv_state=st,
                            hash_args=_hash_args(2), ngram_context=ctx)
    full = oracle.spec_commit(tok, x, qsl, [3, 1], conv_kernel=4, dilation=1, conv_state=st,
                              hash_args=_hash_args(2), ngram_context=ctx)
    lo = oracle.spec_commit(tok, x, qsl, [-5, 0], conv_kernel=4, dilation=1, conv_state=st,
                            hash_args=_hash_args(2), ngram_context=ctx)
    np.testing.assert_array_equal(hi[0], full[0])
    np.testing.assert_array_equal(hi[1], full[1])
    np.testing.assert_array_equal(lo[0], st)
    np.testing.assert_array_equal(lo[1], ctx)


def _random_step(rng, R, N, S, C, max_window):
    lens = rng.integers(0, max_window + 1, size=R)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(qsl[-1])
    x = rng.integers(0, 1 << 16, size=(T, N), dtype=np.uint16)
    tok = rng.integers(1, 1000, size=T, dtype=np.int32)
    st = rng.integers(0, 1 << 16, size=(R, S, N), dtype=np.uint16)
    ctx = rng.integers(1, 1000, size=(R, C), dtype=np.int32)
    acc = rng.integers(0, lens + 1)
    return lens, qsl, x, tok, st, ctx, acc


@pytest.mark.parametrize("seed", range(4))
def test_commit_equals_single_token_decode_steps(seed):
    rng = np.random.default_rng(seed)
    R, N, K, d, C = 5, 8, 4, 2, 3
    S = (K - 1) * d
    lens, qsl, x, tok, st, ctx, acc = _random_step(rng, R, N, S, C, 6)
    so, co = oracle.spec_commit(tok, x, qsl, acc, conv_kernel=K, dilation=d, conv_state=st,
                                hash_args=_hash_args(C), ngram_context=ctx)
    # Feed each request's kept tokens one per decode step, carrying the state.
    w = np.zeros((N, K), np.uint16)
    for r in range(R):
        s_r, c_r = st[r:r + 1], ctx[r:r + 1]
        for i in range(int(acc[r])):
            t = int(qsl[r]) + i
            _, s_r = oracle.conv(x[t:t + 1], [0, 1], w, d, state=s_r, want_state_out=True)
            _, c_r = oracle.ngram_ids(tok[t:t + 1], [0, 1], ngram_context=c_r, want_context_out=True,
                                      **_hash_args(C))
        np.testing.assert_array_equal(so[r], s_r[0])
        np.testing.assert_array_equal(co[r], c_r[0])


def test_accept_all_equals_plain_state_out():
    rng = np.random.default_rng(11)
    R, N, K, d, C = 6, 16, 3, 3, 2
    S = (K - 1) * d
    lens, qsl, x, tok, st, ctx, _ = _random_step(rng, R, N, S, C, 9)
    so, co = oracle.spec_commit(tok, x, qsl, lens, conv_kernel=K, dilation=d, conv_state=st,
                                hash_args=_hash_args(C), ngram_context=ctx)
    w = rng.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    _, so_plain = oracle.conv(x, qsl, w, d, state=st, want_state_out=True)
    _, co_plain = oracle.ngram_ids(tok, qsl, ngram_context=ctx, want_context_out=True, **_hash_args(C))
    np.testing.assert_array_equal(so, so_plain)
    np.testing.assert_array_equal(co, co_plain)


def test_accept_none_null_state_is_zeros_and_eos():
    tok = np.asarray([3, 4], np.int32)
    x = _rows([1, 2])
    so, co = oracle.spec_commit(tok, x, [0, 2], [0], conv_kernel=3, dilation=2, hash_args=_hash_args(3))
    assert so.shape == (1, 4, 8) and not so.any()
    assert co.tolist() == [[EOS] * 3]
