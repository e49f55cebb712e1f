"""Pins for the oracle's n-gram ID function (CPU only).

Definition: "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels",
sections 实现拆解 item 2 and 关键源码片段 (compute_ngram_ids and the ids
kernel).  The oracle is checked against a big-integer brute force, hand-worked
cases under tests/golden/, a textbook closed form, and invariants of the
definition (range, causality, document isolation, request permutation,
chunked == whole).
"""
import json
import os

import numpy as np
import pytest

import bruteforce
import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hash_cases.json")


def _rand_case(rng, *, C=None, hpn=None, with_ctx=None, eos=0, vocab_hi=1000):
    C = C or int(rng.integers(1, 8))
    hpn = hpn or int(rng.integers(1, 4))
    Hfull = C * hpn
    first = int(rng.integers(0, Hfull))
    H = int(rng.integers(1, Hfull - first + 1))
    R = int(rng.integers(1, 6))
    lens = rng.integers(0, 9, size=R)
    qsl = wl.qsl_from_lengths(lens)
    T = int(qsl[-1])
    toks = rng.integers(0, 20, size=T).astype(np.int32)  # small vocab: EOS is frequent
    big = rng.random(T) < 0.3
    toks[big] = rng.integers(0, vocab_hi, size=int(big.sum()))
    mult = rng.integers(-(1 << 63), (1 << 63) - 1, size=(H, C + 1), dtype=np.int64)
    if rng.random() < 0.3:
        mult[:, :] |= 1
    V = rng.integers(2, 5000, size=H).astype(np.int64)
    off = np.concatenate([[0], np.cumsum(V)[:-1]]).astype(np.int64)
    use_ctx = (rng.random() < 0.5) if with_ctx is None else with_ctx
    ctx = rng.integers(0, 20, size=(R, C)).astype(np.int32) if use_ctx else None
    return dict(toks=toks, qsl=qsl, mult=mult, V=V, off=off, C=C, hpn=hpn, first=first, ctx=ctx, eos=eos)


def _oracle(case, want_ctx=True):
    return oracle.ngram_ids(case["toks"], case["qsl"], case["mult"], case["V"], case["off"],
                            context_len=case["C"], heads_per_ngram=case["hpn"], eos_token_id=case["eos"],
                            ngram_context=case["ctx"], first_head=case["first"], want_context_out=want_ctx)


def _brute(case):
    return bruteforce.ngram_ids(case["toks"], case["qsl"], case["mult"], [int(v) for v in case["V"]],
                                [int(o) for o in case["off"]], context_len=case["C"],
                                heads_per_ngram=case["hpn"], eos=case["eos"], context=case["ctx"],
                                first_head=case["first"])


@pytest.mark.parametrize("seed", range(60))
def test_oracle_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    case = _rand_case(rng, eos=int(rng.integers(0, 3)))
    ids, ctx_out = _oracle(case)
    bids, bctx = _brute(case)
    np.testing.assert_array_equal(ids.astype(np.int64), bids)
    np.testing.assert_array_equal(ctx_out.astype(np.int64), bctx.reshape(ctx_out.shape))


def test_golden_hand_cases():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 5
    for c in cases:
        ids, ctx_out = oracle.ngram_ids(
            np.asarray(c["input_ids"]), np.asarray(c["qsl"]), np.asarray(c["multipliers"], dtype=np.int64),
            np.asarray(c["vocab_sizes"]), np.asarray(c["offsets"]), context_len=c["context_len"],
            heads_per_ngram=c["heads_per_ngram"], eos_token_id=c["eos"],
            ngram_context=None if c["context"] is None else np.asarray(c["context"]),
            first_head=c["first_head"], want_context_out=True)
        assert ids.tolist() == c["expected_ids"], c["name"]
        assert ctx_out.tolist() == c["expected_context_out"], c["name"]


def test_range_invariant_cfg3_sized():
    cfg = wl.CONFIGS[3]
    b = wl.make_batch(cfg)
    ids = oracle.ngram_ids(b.input_ids, b.qsl, b.multipliers[0], b.vocab_sizes, b.offsets,
                           context_len=cfg.context_len, heads_per_ngram=cfg.heads_per_ngram,
                           eos_token_id=wl.EOS)
    lo = b.offsets[None, :]
    hi = (b.offsets + b.vocab_sizes)[None, :]
    assert ((ids >= lo) & (ids < hi)).all()


def test_textbook_polynomial_hash():
    # m = (1, B, B^2) and V larger than any sum: ID - off is the base-B polynomial
    B = 1000
    toks = np.asarray([17, 5, 999, 3, 250], dtype=np.int32)
    qsl = np.asarray([0, 5])
    mult = np.asarray([[1, B, 0], [1, B, B * B]], dtype=np.int64)
    V = np.asarray([10 ** 12, 10 ** 12], dtype=np.int64)  # only the oracle: GPU caps V below 2^31
    off = np.asarray([0, 0], dtype=np.int64)
    ids_wide = oracle.ngram_ids(toks, qsl, mult, V, off, context_len=2, heads_per_ngram=1, eos_token_id=0)
    # ids are int32 in storage; the base-B values here stay below 2^31
    seq = [0, 0] + toks.tolist()
    for t in range(len(toks)):
        s0, s1, s2 = seq[t + 2], seq[t + 1], seq[t]
        assert ids_wide[t, 0] == s0 + B * s1
        assert ids_wide[t, 1] == s0 + B * s1 + B * B * s2


def test_fresh_request_start_hashes_eos():
    cfg = wl.CONFIGS[1]
    b = wl.make_batch(cfg)
    ids = oracle.ngram_ids(b.input_ids, b.qsl, b.multipliers[0], b.vocab_sizes, b.offsets,
                           context_len=2, heads_per_ngram=2, eos_token_id=wl.EOS)
    for r in range(b.R):
        a, e = int(b.qsl[r]), int(b.qsl[r + 1])
        if e == a:
            continue
        tok = int(b.input_ids[a])
        for h in range(cfg.H):
            n = 2 + h // 2
            m = [int(x) for x in b.multipliers[0, h]]
            total = tok * m[0]  # every earlier shift is EOS = 0
            want = int(b.offsets[h]) + bruteforce.to_signed64(total) % int(b.vocab_sizes[h])
            assert ids[a, h] == want
            assert n >= 2


def test_context_null_equals_all_eos():
    rng = np.random.default_rng(7)
    case = _rand_case(rng, C=3, hpn=2, with_ctx=False)
    ids0, co0 = _oracle(case)
    case["ctx"] = np.zeros((len(case["qsl"]) - 1, 3), dtype=np.int32)  # EOS = 0
    ids1, co1 = _oracle(case)
    np.testing.assert_array_equal(ids0, ids1)
    np.testing.assert_array_equal(co0, co1)


def test_causality():
    rng = np.random.default_rng(11)
    for _ in range(20):
        case = _rand_case(rng)
        T = len(case["toks"])
        if T < 2:
            continue
        ids, _ = _oracle(case)
        t = int(rng.integers(0, T - 1))
        toks2 = case["toks"].copy()
        toks2[t + 1:] = rng.integers(0, 20, size=T - t - 1)
        ids2, _ = _oracle(dict(case, toks=toks2))
        np.testing.assert_array_equal(ids[: t + 1], ids2[: t + 1])


def test_document_isolation():
    # tokens after an in-request EOS hash exactly like a fresh request starting there
    mult = wl.multipliers(123, 1, 6, 4)[0]
    V = np.asarray(wl.primes_from(5000, 6), dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(V)[:-1]]).astype(np.int64)
    a_part = np.asarray([11, 12, 13, 14], dtype=np.int32)
    b_part = np.asarray([21, 22, 23, 24, 25], dtype=np.int32)
    joined = np.concatenate([a_part, [0], b_part]).astype(np.int32)
    kw = dict(context_len=3, heads_per_ngram=2, eos_token_id=0)
    ids_j = oracle.ngram_ids(joined, [0, len(joined)], mult, V, off, **kw)
    ids_b = oracle.ngram_ids(b_part, [0, len(b_part)], mult, V, off, **kw)
    np.testing.assert_array_equal(ids_j[len(a_part) + 1:], ids_b)


def test_request_permutation_equivariance():
    rng = np.random.default_rng(5)
    for _ in range(10):
        case = _rand_case(rng, with_ctx=True)
        q = case["qsl"]
        R = len(q) - 1
        perm = rng.permutation(R)
        segs = [case["toks"][q[r]:q[r + 1]] for r in range(R)]
        toks_p = np.concatenate([segs[r] for r in perm] + [np.zeros(0, np.int32)]).astype(np.int32)
        q_p = wl.qsl_from_lengths([len(segs[r]) for r in perm])
        ids, co = _oracle(case)
        ids_p, co_p = _oracle(dict(case, toks=toks_p, qsl=q_p, ctx=case["ctx"][perm]))
        rows = [ids[q[r]:q[r + 1]] for r in perm]
        np.testing.assert_array_equal(np.concatenate(rows + [ids[:0]]), ids_p)
        np.testing.assert_array_equal(co[perm], co_p)


def test_chunked_equals_whole():
    # a prefill split into chunks and then one-token decode steps, context carried
    rng = np.random.default_rng(3)
    C, hpn = 3, 2
    mult = wl.multipliers(99, 1, C * hpn, C + 1)[0]
    V = np.asarray(wl.primes_from(100000, C * hpn), dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(V)[:-1]]).astype(np.int64)
    toks = rng.integers(0, 6, size=40).astype(np.int32)  # EOS frequent
    kw = dict(context_len=C, heads_per_ngram=hpn, eos_token_id=0)
    whole, ctx_whole = oracle.ngram_ids(toks, [0, 40], mult, V, off, want_context_out=True, **kw)
    pieces, ctx = [], None
    for lo, hi in [(0, 7), (7, 8), (8, 25), (25, 26), (26, 27), (27, 40)]:
        ids, ctx = oracle.ngram_ids(toks[lo:hi], [0, hi - lo], mult, V, off, ngram_context=ctx,
                                    want_context_out=True, **kw)
        pieces.append(ids)
    np.testing.assert_array_equal(np.concatenate(pieces), whole)
    np.testing.assert_array_equal(ctx, ctx_whole)


def test_empty_requests_and_zero_tokens():
    mult = wl.multipliers(5, 1, 2, 3)[0]
    V = np.asarray([101, 103], dtype=np.int64)
    off = np.asarray([0, 101], dtype=np.int64)
    ctx = np.asarray([[4, 5], [6, 7], [8, 9]], dtype=np.int32)
    ids, co = oracle.ngram_ids(np.zeros(0, np.int32), [0, 0, 0, 0], mult, V, off, context_len=2,
                               heads_per_ngram=1, eos_token_id=0, ngram_context=ctx, want_context_out=True)
    assert ids.shape == (0, 2)
    np.testing.assert_array_equal(co, ctx)  # empty requests carry their context unchanged
    ids, co = oracle.ngram_ids(np.asarray([3], np.int32), [0, 0, 1, 1], mult, V, off, context_len=2,
                               heads_per_ngram=1, eos_token_id=0, ngram_context=ctx, want_context_out=True)
    np.testing.assert_array_equal(co, [[4, 5], [7, 3], [8, 9]])


def test_rejects_bad_arguments():
    mult = np.zeros((2, 3), np.int64)
    with pytest.raises(ValueError):
        oracle.ngram_ids(np.asarray([1, 2], np.int32), [0, 1], mult, [5, 7], [0, 5], context_len=2,
                         heads_per_ngram=1, eos_token_id=0)  # qsl[R] != T
    with pytest.raises(ValueError):
        oracle.ngram_ids(np.asarray([1], np.int32), [0, 1], mult, [0, 7], [0, 5], context_len=2,
                         heads_per_ngram=1, eos_token_id=0)  # V_h <= 0
