"""GPU parity of every libple entry point against the oracle, at sizes the
oracle finishes in seconds (several tiles plus ragged tails) and on the edge
cases of the method.  IDs, rows and fp8 dequant: bit-exact.  kv_proj: within
the fp32 dot-product error bound plus one bf16 ulp (one ulp wherever the value
is not cancelled to near zero).  Gate and conv bf16 outputs: max-abs 2e-2 (and
at most one bf16 ulp in practice); the fp32 gate value: rel 1e-5."""
import json
import os

import numpy as np
import pytest
import torch

import layer_embedding_lookup_amd as ple
import oracle
import workloads as wl
from gpu_util import (DEV, bf16_f64, bf16_ulp_distance, check_gate_conv_stages, dev, dev_bf16, hash_params,
                      host_bits, last_rows_of_requests, log, oracle_ids)

pytestmark = pytest.mark.gpu

GATE_ABS_TOL = 2e-2
CONV_ABS_TOL = 2e-2
GATE_REL_TOL = 1e-5


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    log(f"device: {torch.cuda.get_device_name(0)}; {ple.ple_version()}")


# ------------------------------------------------------------------ ids

@pytest.mark.parametrize("cfg_idx", [1, 2, 3, 4, 5])
def test_ids_parity_configs(cfg_idx):
    cfg = wl.CONFIGS[cfg_idx]
    b = wl.make_batch(cfg, layers=2)
    for layer in range(2):
        log(f"ids cfg{cfg_idx} layer{layer} T={cfg.T} R={b.R} H={cfg.H}")
        want, want_ctx = oracle_ids(b, layer, want_context_out=True)
        ctx_d = dev(b.ngram_context) if b.ngram_context is not None else None
        ctx_out = torch.full((b.R, cfg.context_len), -1, dtype=torch.int32, device=DEV)
        got = ple.ple_ngram_ids(hash_params(b, layer), dev(b.input_ids), dev(b.qsl), ngram_context=ctx_d,
                                ngram_context_out=ctx_out)
        np.testing.assert_array_equal(got.cpu().numpy(), want)
        np.testing.assert_array_equal(ctx_out.cpu().numpy(), want_ctx)


def test_ids_cfg1_with_context():
    b = wl.make_batch(wl.CONFIGS[1], with_context=True)
    want = oracle_ids(b)
    got = ple.ple_ngram_ids(hash_params(b), dev(b.input_ids), dev(b.qsl), ngram_context=dev(b.ngram_context))
    np.testing.assert_array_equal(got.cpu().numpy(), want)


def _random_case(rng):
    C = int(rng.integers(1, 8))
    hpn = int(rng.integers(1, 5))
    Hfull = min(C * hpn, 32)
    first = int(rng.integers(0, Hfull))
    H = int(rng.integers(1, min(Hfull - first, 32) + 1))
    R = int(rng.integers(1, 40))
    lens = rng.integers(0, 30, size=R)
    lens[rng.random(R) < 0.2] = 0
    qsl = wl.qsl_from_lengths(lens)
    T = int(qsl[-1])
    eos = int(rng.integers(0, 3))
    toks = rng.integers(0, 12, size=T).astype(np.int32)  # EOS frequent
    big = rng.random(T) < 0.4
    toks[big] = rng.integers(0, 2 ** 31 - 1, size=int(big.sum()))
    mult = rng.integers(-(1 << 63), (1 << 63) - 1, size=(H, C + 1), dtype=np.int64)
    V = rng.integers(1, 2 ** 31 // 40, size=H).astype(np.int64)
    V[rng.random(H) < 0.2] = 1
    off = np.concatenate([[0], np.cumsum(V)[:-1]]).astype(np.int64)
    ctx = rng.integers(0, 12, size=(R, C)).astype(np.int32) if rng.random() < 0.5 else None
    return dict(C=C, hpn=hpn, first=first, H=H, qsl=qsl, toks=toks, eos=eos, mult=mult, V=V, off=off, ctx=ctx)


@pytest.mark.parametrize("seed", range(40))
def test_ids_edge_random(seed):
    rng = np.random.default_rng(1000 + seed)
    c = _random_case(rng)
    R = len(c["qsl"]) - 1
    log(f"ids edge seed={seed} T={len(c['toks'])} R={R} C={c['C']} H={c['H']} first={c['first']}")
    want, want_ctx = oracle.ngram_ids(c["toks"], c["qsl"], c["mult"], c["V"], c["off"], context_len=c["C"],
                                      heads_per_ngram=c["hpn"], eos_token_id=c["eos"], ngram_context=c["ctx"],
                                      first_head=c["first"], want_context_out=True)
    hp = ple.HashParams(c["mult"], c["V"], c["off"], heads_per_ngram=c["hpn"], context_len=c["C"],
                        eos_token_id=c["eos"], first_head=c["first"])
    ctx_out = torch.full((R, c["C"]), -7, dtype=torch.int32, device=DEV)
    toks = dev(c["toks"]) if len(c["toks"]) else torch.zeros(0, dtype=torch.int32, device=DEV)
    got = ple.ple_ngram_ids(hp, toks, dev(c["qsl"]), ngram_context=None if c["ctx"] is None else dev(c["ctx"]),
                            ngram_context_out=ctx_out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), want)
    np.testing.assert_array_equal(ctx_out.cpu().numpy(), want_ctx)


def test_ids_and_rows_beyond_1024_requests():
    """More than 1024 requests: the request search falls back from the query_start_loc probe to a
    binary search (IDs, context out and rows against the oracle; 1500 requests of 0-8 tokens, a third of
    them empty, with carried context)."""
    rng = np.random.default_rng(77)
    R, C, hpn = 1500, 2, 2
    lens = rng.integers(0, 9, size=R)
    lens[rng.random(R) < 0.33] = 0
    qsl = wl.qsl_from_lengths(lens)
    T = int(qsl[-1])
    H = C * hpn
    toks = rng.integers(0, 151936, size=T).astype(np.int32)
    mult = rng.integers(-(1 << 63), (1 << 63) - 1, size=(H, C + 1), dtype=np.int64)
    V = np.asarray([997, 1009, 1013, 1019], dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(V)[:-1]]).astype(np.int64)
    ctx = rng.integers(0, 151936, size=(R, C)).astype(np.int32)
    log(f"ids beyond 1024 requests: R={R} T={T}")
    want, want_ctx = oracle.ngram_ids(toks, qsl, mult, V, off, context_len=C, heads_per_ngram=hpn,
                                      eos_token_id=wl.EOS, ngram_context=ctx, want_context_out=True)
    hp = ple.HashParams(mult, V, off, heads_per_ngram=hpn, context_len=C, eos_token_id=wl.EOS)
    ctx_out = torch.full((R, C), -7, dtype=torch.int32, device=DEV)
    got = ple.ple_ngram_ids(hp, dev(toks), dev(qsl), ngram_context=dev(ctx), ngram_context_out=ctx_out)
    np.testing.assert_array_equal(got.cpu().numpy(), want)
    np.testing.assert_array_equal(ctx_out.cpu().numpy(), want_ctx)
    table = wl.normal_bf16((int(V.sum()), 64), 78, 0.02)
    rows = ple.ple_lookup(hp, ple.Table.from_tensor(dev_bf16(table)), dev(toks), dev(qsl), ngram_context=dev(ctx))
    np.testing.assert_array_equal(host_bits(rows), oracle.gather_bf16(table, want).reshape(T, -1))


@pytest.mark.parametrize("seed", range(24))
@pytest.mark.parametrize("fmt", ["bf16-32", "bf16-512", "fp8-512", "nvfp4-512"])
def test_lookup_edge_random(seed, fmt):
    """The fused lookup on the random edge batches (orders up to 8, head shards of up to 32 heads, empty
    and one-token requests, frequent EOS, carried context), with vocabularies small enough for a real
    table: its IDs (ids_out) and rows bit-exact against the oracle.  Rows of 512 elements take the
    scalar-address row stream for fp8 and NVFP4 (ragged last passes included), the per-lane stream for
    bf16; 32-element rows the per-lane stream."""
    rng = np.random.default_rng(5000 + seed)
    c = _random_case(rng)
    H, T = c["H"], len(c["toks"])
    c["V"] = rng.integers(1, 700, size=H).astype(np.int64)
    c["off"] = np.concatenate([[0], np.cumsum(c["V"])[:-1]]).astype(np.int64)
    nrows = int(c["V"].sum())
    R = len(c["qsl"]) - 1
    log(f"lookup edge {fmt} seed={seed} T={T} R={R} C={c['C']} H={H} first={c['first']}")
    want_ids = oracle.ngram_ids(c["toks"], c["qsl"], c["mult"], c["V"], c["off"], context_len=c["C"],
                                heads_per_ngram=c["hpn"], eos_token_id=c["eos"], ngram_context=c["ctx"],
                                first_head=c["first"])
    kind, D = fmt.split("-")[0], int(fmt.split("-")[1])
    if kind == "bf16":
        table = rng.integers(0, 65536, size=(nrows, D), dtype=np.uint16)
        tb, keep = ple.Table.from_tensor(dev_bf16(table)), None
        want = table[want_ids.reshape(-1)] if T else np.zeros((0, D), np.uint16)
    elif kind == "fp8":
        codes = rng.integers(0, 256, size=(nrows, D), dtype=np.uint8)
        scales = np.exp(rng.uniform(-8, 8, nrows)).astype(np.float32)
        keep = (dev(codes), dev(scales))
        tb = ple.Table.from_tensor(*keep)
        want = oracle.gather_fp8(codes, scales, want_ids)
    else:
        codes = rng.integers(0, 256, size=(nrows, D // 2), dtype=np.uint8)
        bsc = rng.integers(0, 256, size=(nrows, D // 16), dtype=np.uint8)
        tsc = np.asarray([0.37], np.float32)
        keep = (dev(codes), dev(bsc), dev(tsc))
        tb = ple.Table.nvfp4(*keep)
        want = oracle.gather_nvfp4(codes, bsc, tsc[0], want_ids)
    hp = ple.HashParams(c["mult"], c["V"], c["off"], heads_per_ngram=c["hpn"], context_len=c["C"],
                        eos_token_id=c["eos"], first_head=c["first"])
    toks = dev(c["toks"]) if T else torch.zeros(0, dtype=torch.int32, device=DEV)
    ids_out = torch.full((T, H), -1, dtype=torch.int32, device=DEV)
    rows = ple.ple_lookup(hp, tb, toks, dev(c["qsl"]), ngram_context=None if c["ctx"] is None else dev(c["ctx"]),
                          ids_out=ids_out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids_out.cpu().numpy(), want_ids)
    np.testing.assert_array_equal(host_bits(rows).reshape(-1, D), want.reshape(-1, D))


def test_ids_golden_cases():
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hash_cases.json")))["cases"]
    for c in cases:
        log(f"golden {c['name']}")
        hp = ple.HashParams(np.asarray(c["multipliers"], np.int64), c["vocab_sizes"], c["offsets"],
                            heads_per_ngram=c["heads_per_ngram"], context_len=c["context_len"],
                            eos_token_id=c["eos"], first_head=c["first_head"])
        ctx = None if c["context"] is None else dev(np.asarray(c["context"], np.int32))
        ctx_out = torch.empty((len(c["qsl"]) - 1, c["context_len"]), dtype=torch.int32, device=DEV)
        got = ple.ple_ngram_ids(hp, dev(np.asarray(c["input_ids"], np.int32)), dev(np.asarray(c["qsl"], np.int32)),
                                ngram_context=ctx, ngram_context_out=ctx_out)
        assert got.cpu().tolist() == c["expected_ids"], c["name"]
        assert ctx_out.cpu().tolist() == c["expected_context_out"], c["name"]


def test_ids_empty_batch_carries_context():
    hp = ple.HashParams(np.ones((2, 3), np.int64), [11, 13], [0, 11], heads_per_ngram=1, context_len=2,
                        eos_token_id=0)
    ctx = dev(np.asarray([[4, 5], [6, 7], [8, 9]], np.int32))
    ctx_out = torch.zeros((3, 2), dtype=torch.int32, device=DEV)
    got = ple.ple_ngram_ids(hp, torch.zeros(0, dtype=torch.int32, device=DEV), dev(np.zeros(4, np.int32)),
                            ngram_context=ctx, ngram_context_out=ctx_out)
    assert got.shape == (0, 2)
    assert ctx_out.cpu().tolist() == [[4, 5], [6, 7], [8, 9]]


def test_ids_context_null_equals_all_eos():
    b = wl.make_batch(wl.CONFIGS[2])
    hp = hash_params(b)
    a = ple.ple_ngram_ids(hp, dev(b.input_ids), dev(b.qsl))
    z = ple.ple_ngram_ids(hp, dev(b.input_ids), dev(b.qsl),
                          ngram_context=torch.zeros((b.R, 2), dtype=torch.int32, device=DEV))
    assert torch.equal(a, z)


def test_ids_chunked_equals_whole_on_gpu():
    cfg = wl.CONFIGS[3]
    b = wl.make_batch(cfg)
    hp = hash_params(b)
    qsl = b.qsl
    r = int(np.argmax(np.diff(qsl)))  # the longest request
    a0, a1 = int(qsl[r]), int(qsl[r + 1])
    toks = b.input_ids[a0:a1]
    whole = ple.ple_ngram_ids(hp, dev(toks), dev(np.asarray([0, len(toks)], np.int32)))
    ctx = None
    parts = []
    cuts = sorted({0, 1, 5, len(toks) // 3, len(toks) // 3 + 1, len(toks) - 1, len(toks)})
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        out_ctx = torch.empty((1, 2), dtype=torch.int32, device=DEV)
        parts.append(ple.ple_ngram_ids(hp, dev(toks[lo:hi]), dev(np.asarray([0, hi - lo], np.int32)),
                                       ngram_context=ctx, ngram_context_out=out_ctx))
        ctx = out_ctx
    assert torch.equal(torch.cat(parts), whole)


# ------------------------------------------------------------------ lookup / gather

def _table_dev(cfg, seed=None):
    q, sc = wl.make_table(cfg, seed=seed)
    if cfg.table_dtype == "bf16":
        t = dev_bf16(q)
        return q, sc, ple.Table.from_tensor(t), (t,)
    qt, st = dev(q), dev(sc)
    return q, sc, ple.Table.from_tensor(qt, st), (qt, st)


@pytest.mark.parametrize("cfg_idx", [1, 2])
def test_lookup_parity_small_configs(cfg_idx):
    cfg = wl.CONFIGS[cfg_idx]
    b = wl.make_batch(cfg, layers=2)
    table, _, tb, keep = _table_dev(cfg)
    for layer in range(2):
        log(f"lookup cfg{cfg_idx} layer{layer}")
        ids = oracle_ids(b, layer)
        want = oracle.gather_bf16(table, ids).reshape(cfg.T, -1)
        ids_out = torch.empty((cfg.T, cfg.H), dtype=torch.int32, device=DEV)
        ctx = dev(b.ngram_context) if b.ngram_context is not None else None
        rows = ple.ple_lookup(hash_params(b, layer), tb, dev(b.input_ids), dev(b.qsl), ngram_context=ctx,
                              ids_out=ids_out)
        np.testing.assert_array_equal(ids_out.cpu().numpy(), ids)
        np.testing.assert_array_equal(host_bits(rows), want)
        rows2 = ple.ple_gather(tb, dev(ids))
        np.testing.assert_array_equal(host_bits(rows2), want)


def _small_fp8_cfg():
    base = wl.CONFIGS[4]
    import dataclasses
    return dataclasses.replace(base, idx=40, T=700, vocab_base=5003)


def test_lookup_fp8_small():
    cfg = _small_fp8_cfg()
    b = wl.make_batch(cfg)
    q, sc, tb, keep = _table_dev(cfg)
    ids = oracle_ids(b)
    want = oracle.gather_fp8(q, sc, ids).reshape(cfg.T, -1)
    rows = ple.ple_lookup(hash_params(b), tb, dev(b.input_ids), dev(b.qsl))
    np.testing.assert_array_equal(host_bits(rows), want)


def test_fp8_every_code_and_scale():
    rng = np.random.default_rng(8)
    D, nrows = 256, 64
    codes = np.stack([rng.permutation(256) for _ in range(nrows)]).astype(np.uint8)
    scales = np.exp(rng.uniform(-40, 40, nrows)).astype(np.float32)
    scales[:4] = [1.0, 2.0 ** -20, 3.0e30, 1e-38]
    ids = rng.integers(0, nrows, size=(50, 3)).astype(np.int32)
    want = oracle.gather_fp8(codes, scales, ids).reshape(50, -1)
    tb = ple.Table.from_tensor(dev(codes), dev(scales))
    rows = ple.ple_gather(tb, dev(ids))
    np.testing.assert_array_equal(host_bits(rows), want)


@pytest.mark.parametrize("D", [32, 256, 512, 40])
def test_gather_bf16_dims_and_clamping(D):
    rng = np.random.default_rng(D)
    nrows = 3000
    table = rng.integers(0, 65536, size=(nrows, D), dtype=np.uint16)
    ids = rng.integers(0, nrows, size=(333, 5)).astype(np.int32)
    ids[0, 0], ids[1, 1], ids[2, 2] = -5, nrows, 2 ** 31 - 1   # clamped into [0, rows)
    clamped = np.clip(ids, 0, nrows - 1)
    tb = ple.Table.from_tensor(dev_bf16(table))
    rows = ple.ple_gather(tb, dev(ids))
    np.testing.assert_array_equal(host_bits(rows), table[clamped.reshape(-1)].reshape(333, -1))


def test_lookup_head_subset_matches_full():
    cfg = wl.CONFIGS[2]
    b = wl.make_batch(cfg)
    table, _, tb, keep = _table_dev(cfg)
    full = ple.ple_lookup(hash_params(b), tb, dev(b.input_ids), dev(b.qsl), ngram_context=dev(b.ngram_context))
    D = cfg.D
    for first, H in [(0, 4), (4, 4), (3, 2), (7, 1)]:
        part = ple.ple_lookup(hash_params(b, first_head=first, num_heads=H), tb, dev(b.input_ids), dev(b.qsl),
                              ngram_context=dev(b.ngram_context))
        assert torch.equal(part, full.view(cfg.T, cfg.H, D)[:, first:first + H].reshape(cfg.T, -1))


# ------------------------------------------------------------------ kv_proj

def _check_kv(got, want, x, w):
    """fp32 accumulation of K products, then one bf16 rounding: the error bound
    is gamma_K * sum_k |x_k w_k| (gamma_K = K u / (1 - K u), u = 2^-24) plus one
    bf16 ulp of the result.  Near zero (cancellation) this is what limits the
    error; elsewhere the results are the correctly rounded value or a neighbour."""
    K = x.shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    absdot = bf16_f64(oracle.kv_proj(x & np.uint16(0x7FFF), w & np.uint16(0x7FFF))) * 1.01
    g, e = bf16_f64(got), bf16_f64(want)
    ulp = np.maximum(np.abs(e), 2.0 ** -126) * 2.0 ** -7
    assert (np.abs(g - e) <= gamma * absdot + ulp).all()
    d = bf16_ulp_distance(got, want)
    big = np.abs(e) > 1e-2
    assert d[big].max() <= 1
    assert (d > 0).mean() < 0.01


@pytest.mark.parametrize("M,K,O", [# 64 x 64 tile kernel (< 256 tiles of 128 x 128), incl. one K-slice
                                   (24, 128, 256), (1, 64, 16), (300, 192, 80), (129, 128, 144), (200, 64, 272),
                                   (256, 2048, 4096), (1000, 512, 1024), (65, 64, 4096),
                                   # 128 x 128 tiles: the speculative-verify width, ragged in M and O
                                   (1024, 2048, 4096), (1000, 2048, 4112), (2048, 64, 2064),
                                   # 256 x 256 tile kernel (>= 256 tiles): 1 to 5 K-slices of 64,
                                   # ragged in M and in O
                                   (4100, 128, 4112), (4103, 256, 4096), (64, 64, 65536), (2048, 192, 8192),
                                   (2100, 320, 8208),
                                   # 512 and more 256 x 256 tiles (two or more per CU): whole tiles, an
                                   # uneven 522-tile split
                                   (4096, 704, 8192), (4608, 768, 7424), (8192, 1024, 4096)])
def test_kv_proj_parity(M, K, O):
    log(f"kv_proj M={M} K={K} O={O}")
    x = wl.normal_bf16((M, K), 100 + M, 0.02)
    w = wl.normal_bf16((O, K), 200 + O, 12.5 / np.sqrt(K))
    got = host_bits(ple.ple_kv_proj(dev_bf16(x), dev_bf16(w)))
    if M * O * K > 4e9:
        # the oracle takes the first and last rows (ragged tile edge) and a seeded sample
        rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(M - 40, M),
                                         np.random.default_rng(M).integers(0, M, 40)]))
        _check_kv(got[rows], oracle.kv_proj(x[rows], w), x[rows], w)
    else:
        _check_kv(got, oracle.kv_proj(x, w), x, w)


def test_kv_proj_sampled_rows_at_prefill_shape():
    cfg = wl.CONFIGS[3]
    M, K, O = cfg.T, cfg.H * cfg.D, 2 * cfg.N
    x = wl.normal_bf16((M, K), 5, 0.02)
    w = wl.make_kv_weight(cfg)
    got = host_bits(ple.ple_kv_proj(dev_bf16(x), dev_bf16(w)))
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(M - 64, M),
                                     np.random.default_rng(0).integers(0, M, 64)]))
    want = oracle.kv_proj(x[rows], w)
    _check_kv(got[rows], want, x[rows], w)


# ------------------------------------------------------------------ gate

@pytest.mark.parametrize("T,N", [(24, 128), (256, 2048), (333, 4096), (5, 8), (7, 4104)])
def test_gate_parity(T, N):
    log(f"gate T={T} N={N}")
    h = wl.normal_bf16((T, N), 300 + N, 1.0)
    kv = wl.normal_bf16((T, 2 * N), 400 + N, 0.25)
    want, g_want = oracle.gate(h, kv, 1e-6)
    out, g = ple.ple_gate(dev_bf16(h), dev_bf16(kv), eps=1e-6)
    got = host_bits(out)
    assert np.abs(bf16_f64(got) - bf16_f64(want)).max() <= GATE_ABS_TOL
    assert bf16_ulp_distance(got, want).max() <= 1
    gg = g.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(gg, g_want, rtol=GATE_REL_TOL, atol=0)
    assert ((gg > 0) & (gg < 1)).all()


def test_gate_closed_forms_on_gpu():
    N = 256
    h = np.zeros((2, N))
    h[:, ::2] = 1.0
    k = np.zeros((2, N))
    k[:, 1::2] = -0.75
    v = np.linspace(-1, 1, N)[None].repeat(2, 0)
    bits = lambda a: np.asarray([oracle.bf16_from_double(float(x)) for x in a.ravel()], np.uint16).reshape(a.shape)
    out, g = ple.ple_gate(dev_bf16(bits(h)), dev_bf16(np.concatenate([bits(k), bits(v)], 1)))
    assert (g.cpu().numpy() == 0.5).all()
    np.testing.assert_array_equal(bf16_f64(host_bits(out)), bf16_f64(bits(v)) / 2)


# ------------------------------------------------------------------ conv

CONV_CASES = [
    # (lengths, N, K, d, with_state)
    ([7, 1, 13, 3], 128, 4, 2, False),
    ([7, 1, 13, 3], 128, 4, 2, True),
    ([1] * 64, 2048, 4, 3, True),
    ([0, 5, 0, 0, 40, 1, 0], 64, 3, 5, True),
    ([50, 20], 64, 1, 1, False),
    ([33, 0, 9], 72, 7, 2, True),   # kernel size 7: the LDS-staged tile kernel
    ([100], 16, 2, 9, True),
    # the generic kernel (any kernel size, any span): kernel sizes above 8,
    # spans above 64 rows, and weights wider than 64 KiB with a span above 64
    ([30, 0, 17, 1], 16, 12, 2, True),
    ([25, 3, 0, 40], 24, 6, 13, True),
    ([9, 70, 1], 8200, 4, 22, True),
    ([5, 90], 64, 16, 1, False),
    # long requests (at least 4 d tokens each on average): the sliding-window
    # kernel, with requests shorter than the dilation, empty requests, a
    # partly filled last channel slice (N = 520) and kernel sizes 1-4
    ([300, 1, 0, 257, 2, 140], 4096, 4, 3, True),
    ([300, 1, 0, 257, 2, 140], 520, 3, 2, False),
    ([500], 256, 2, 5, True),
    ([97, 64, 161], 128, 1, 4, True),
    ([1000, 23], 64, 4, 1, True),
    # the LDS-staged kernel's request search at 64 requests and more (the query_start_loc probe of up
    # to 1024 requests, then the binary search beyond): 100 requests of 8-32 tokens, 1100 of 16
    (list(range(8, 33)) * 4, 256, 4, 3, True),
    ([16] * 1100, 64, 4, 3, True),
    # the per-row kernel (decode-shaped: about one token per request) beyond 1024 requests
    ([1] * 1100 + [2, 0, 3], 256, 4, 3, True),
]


@pytest.mark.parametrize("case", range(len(CONV_CASES)))
def test_conv_parity(case):
    lens, N, K, d, with_state = CONV_CASES[case]
    log(f"conv case {case}: R={len(lens)} N={N} K={K} d={d} state={with_state}")
    qsl = wl.qsl_from_lengths(lens)
    T, R, S = int(qsl[-1]), len(lens), (K - 1) * d
    x = wl.normal_bf16((T, N), 500 + case, 0.5)
    w = wl.uniform_bf16((N, K), 600 + case, -0.5, 0.5)
    st = wl.normal_bf16((R, S, N), 700 + case, 0.125) if with_state and S > 0 else None
    want, st_want = oracle.conv(x, qsl, w, d, state=st, want_state_out=True)
    st_out = torch.empty((R, S, N), dtype=torch.bfloat16, device=DEV) if S > 0 else None
    xd = dev_bf16(x) if T else torch.zeros((0, N), dtype=torch.bfloat16, device=DEV)
    y = ple.ple_conv(xd, dev(qsl), dev_bf16(w), dilation=d, conv_state=None if st is None else dev_bf16(st),
                     conv_state_out=st_out)
    got = host_bits(y)
    assert np.abs(bf16_f64(got) - bf16_f64(want)).max() <= CONV_ABS_TOL
    assert bf16_ulp_distance(got, want).max() <= 1
    if S > 0:
        np.testing.assert_array_equal(host_bits(st_out), st_want)


def test_conv_chunked_equals_whole_on_gpu():
    N, K, d = 256, 4, 3
    x = wl.normal_bf16((200, N), 801, 0.5)
    w = wl.uniform_bf16((N, K), 802, -0.5, 0.5)
    S = (K - 1) * d
    whole = ple.ple_conv(dev_bf16(x), dev(np.asarray([0, 200], np.int32)), dev_bf16(w), dilation=d)
    st = None
    parts = []
    for lo, hi in [(0, 3), (3, 4), (4, 120), (120, 121), (121, 200)]:
        so = torch.empty((1, S, N), dtype=torch.bfloat16, device=DEV)
        parts.append(ple.ple_conv(dev_bf16(x[lo:hi]), dev(np.asarray([0, hi - lo], np.int32)), dev_bf16(w),
                                  dilation=d, conv_state=st, conv_state_out=so))
        st = so
    assert torch.equal(torch.cat(parts), whole)


# ------------------------------------------------------------------ fused prefill

def _layer(cfg, b, layer=0):
    table, scales, tb, keep = _table_dev(cfg)
    kvw = wl.make_kv_weight(cfg, layer=layer)
    cw = wl.make_conv_weight(cfg)
    L = ple.Layer(hash_params(b, layer), tb, dev_bf16(kvw), dev_bf16(cw), conv_dilation=cfg.conv_dilation,
                  eps=cfg.eps)
    return L, table, scales, kvw, cw, keep


def _oracle_chain(cfg, b, table, scales, kvw, cw, hidden, tokens=None, layer=0):
    args = dict(input_ids=b.input_ids, qsl=b.qsl, multipliers=b.multipliers[layer], vocab_sizes=b.vocab_sizes,
                offsets=b.offsets, context_len=cfg.context_len, heads_per_ngram=cfg.heads_per_ngram,
                eos_token_id=wl.EOS, ngram_context=b.ngram_context)
    return oracle.prefill(args, table, scales, hidden, kvw, cw, cfg.conv_dilation, qsl=b.qsl, eps=cfg.eps,
                          conv_state=b.conv_state, tokens=tokens)


@pytest.mark.parametrize("variant", ["cfg1", "cfg1-ctx-state", "cfg2", "cfg1-long-state", "cfg1-k7-d2",
                                     "cfg1-k12-d1", "cfg1-many-requests"])
def test_prefill_fused_parity_small(variant):
    """The whole chain against the oracle's chain (out within 2e-2), and each stage against the oracle
    run on the GPU's own input to it: kv_proj on the gathered rows, the fp32 gate at rel 1e-5 on the
    GPU's kv (read from the workspace), the conv on the GPU's conv input.  Conv kernels above 4 take the
    entry point's other tail: the gate writes the gated value in full and the generic conv reads it."""
    import dataclasses
    cfg = wl.CONFIGS[2 if variant == "cfg2" else 1]
    if variant == "cfg1-long-state":
        # long requests: the conv walks each residue class with a sliding window
        cfg = dataclasses.replace(cfg, idx=43, T=400, requests="fixed", fixed_lengths=(150, 1, 0, 97, 2, 150))
    if variant.startswith("cfg1-k"):
        K, d = int(variant.split("-k")[1].split("-")[0]), int(variant.split("-d")[1])
        cfg = dataclasses.replace(cfg, idx=90 + K, conv_kernel=K, conv_dilation=d)
    if variant == "cfg1-many-requests":
        # 1100 requests of 0-2 tokens: the lookup's and the per-row conv's request searches fall back to
        # a binary search beyond 1024 requests; every request carries context and conv state
        lens = tuple(int(x) for x in np.random.default_rng(44).integers(0, 3, size=1100))
        cfg = dataclasses.replace(cfg, idx=44, T=sum(lens), requests="fixed", fixed_lengths=lens)
    if variant in ("cfg1-ctx-state", "cfg1-long-state", "cfg1-many-requests") or variant.startswith("cfg1-k"):
        b = wl.make_batch(cfg, with_context=True, with_state=True)
    else:
        b = wl.make_batch(cfg)
    log(f"prefill {variant}")
    L, table, scales, kvw, cw, keep = _layer(cfg, b)
    hidden = wl.make_hidden(cfg)
    ref = _oracle_chain(cfg, b, table, scales, kvw, cw, hidden)
    S = cfg.S
    st_out = torch.empty((b.R, S, cfg.N), dtype=torch.bfloat16, device=DEV)
    ctx_out = torch.empty((b.R, cfg.context_len), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.T,), dtype=torch.float32, device=DEV)
    ws = torch.empty((ple.ple_prefill_workspace_bytes(L, cfg.T),), dtype=torch.uint8, device=DEV)
    out = ple.ple_prefill_fused(L, dev(b.input_ids), dev(b.qsl), dev_bf16(hidden),
                                ngram_context=None if b.ngram_context is None else dev(b.ngram_context),
                                ngram_context_out=ctx_out,
                                conv_state=None if b.conv_state is None else dev_bf16(b.conv_state),
                                conv_state_out=st_out, gate=gate, workspace=ws)
    got = host_bits(out)
    assert np.abs(bf16_f64(got) - bf16_f64(ref["y"])).max() <= CONV_ABS_TOL
    _, want_ctx = oracle_ids(b, want_context_out=True)
    np.testing.assert_array_equal(ctx_out.cpu().numpy(), want_ctx)
    kv_gpu = host_bits(ple.prefill_kv(L, ws, cfg.T))
    _check_kv(kv_gpu, ref["kv"], ref["rows"], kvw)
    written = last_rows_of_requests(b.qsl, cfg.S, cfg.T)
    gated_ws = host_bits(ple.prefill_conv_input(L, ws, cfg.T))
    check_gate_conv_stages(hidden, kv_gpu, gate.cpu().numpy(), gated_ws, got, b.qsl, cw, cfg.conv_dilation, cfg.eps,
                           conv_state=b.conv_state, state_out_gpu=host_bits(st_out), gated_rows=written)
    # the carried state is a copy of the conv inputs the GPU left in the workspace
    _, st_copy = oracle.conv(np.where(written[:, None], gated_ws, 0).astype(np.uint16), b.qsl, cw, cfg.conv_dilation,
                             state=b.conv_state, want_state_out=True)
    np.testing.assert_array_equal(host_bits(st_out), st_copy)


def _run_fused_both(cfg, b, L, hidden, *, with_ctx, with_state, max_request_tokens, T=None):
    """One ple_prefill_fused call; returns out, gate, conv input, state out and context out (host)."""
    T = cfg.T if T is None else T
    S = (L.conv_weight.shape[1] - 1) * L.conv_dilation
    st_out = torch.full((b.R, S, cfg.N), 7.0, dtype=torch.bfloat16, device=DEV)
    ctx_out = torch.full((b.R, cfg.context_len), -3, dtype=torch.int32, device=DEV)
    gate = torch.full((T,), -1.0, dtype=torch.float32, device=DEV)
    ws = torch.zeros((ple.ple_prefill_workspace_bytes(L, T),), dtype=torch.uint8, device=DEV)
    toks = dev(b.input_ids) if T else torch.zeros(0, dtype=torch.int32, device=DEV)
    out = ple.ple_prefill_fused(L, toks, dev(b.qsl), dev_bf16(hidden),
                                ngram_context=dev(b.ngram_context) if with_ctx else None, ngram_context_out=ctx_out,
                                conv_state=dev_bf16(b.conv_state) if with_state else None, conv_state_out=st_out,
                                gate=gate, workspace=ws, max_request_tokens=max_request_tokens)
    torch.cuda.synchronize()
    return (host_bits(out), gate.cpu().numpy(), host_bits(ple.prefill_conv_input(L, ws, T)), host_bits(st_out),
            ctx_out.cpu().numpy(), host_bits(ple.prefill_kv(L, ws, T)))


@pytest.mark.parametrize("case", ["decode-256", "decode-256-fresh", "tiny-empty-requests-k4", "tiny-k1", "tiny-k2",
                                  "tiny-k3-fresh", "all-empty", "windows-256x4", "windows-256x4-fresh",
                                  "tiny-windows-k4-d2", "tiny-windows-k2-d1", "tiny-windows-k3-d1-fresh",
                                  "tiny-windows-k4-d3", "tiny-many-k4"])
def test_decode_tail_equals_plain_path(case):
    """With max_request_tokens = 1..4 (decode steps, speculative verify windows) the fused entry point
    runs gate, conv and the carried state and context as one kernel; every output is the same bits as
    the separate kernels' (same arithmetic), including the conv input left in the workspace, on
    batches of one-token, window and empty requests (taps inside and before the window)."""
    import dataclasses
    hint = 4 if "windows" in case else 1
    if case.startswith("decode-256") or case.startswith("windows-256"):
        cfg = wl.CONFIGS[2]
        b = wl.make_batch(cfg, with_context=True, with_state=True)
        K = cfg.conv_kernel
        if case.startswith("windows"):
            W = 4
            cfg = dataclasses.replace(cfg, T=cfg.T * W)
            b = dataclasses.replace(b, cfg=cfg, input_ids=wl.make_tokens(cfg, T=cfg.T),
                                    qsl=np.arange(0, cfg.T + 1, W, dtype=np.int32))
    else:
        base = wl.CONFIGS[1]
        K = int(case.split("-k")[1][0]) if "-k" in case else 4
        d = int(case.split("-d")[1][0]) if "-d" in case else base.conv_dilation
        rng = np.random.default_rng(61 + K + 7 * d)
        if case == "all-empty":
            lens = [0, 0, 0]
        elif "many" in case:
            # 1100 requests of 0 or 1 tokens: past the 1024 requests the plain path's searches probe
            lens = [int(x) for x in rng.integers(0, 2, size=1100)]
        elif "windows" in case:
            lens = [int(x) for x in rng.integers(0, 5, size=12)]
            lens[0], lens[1] = 4, 0
        else:
            lens = [1, 0, 1, 1, 0, 0, 1, 1, 0, 1]
        cfg = dataclasses.replace(base, idx=60, T=int(sum(lens)), conv_kernel=K, conv_dilation=d)
        b = wl.make_batch(base, with_context=True, with_state=True)
        R = len(lens)
        qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        S = (K - 1) * cfg.conv_dilation
        b = dataclasses.replace(b, cfg=cfg, input_ids=rng.integers(0, 1000, size=cfg.T).astype(np.int32), qsl=qsl,
                                ngram_context=rng.integers(0, 1000, size=(R, cfg.context_len)).astype(np.int32),
                                conv_state=wl.normal_bf16((R, S, cfg.N), 62, 0.125))
    fresh = case.endswith("fresh")
    table, scales, tb, keep = _table_dev(cfg)
    kvw = wl.make_kv_weight(cfg)
    cw = wl.normal_bf16((cfg.N, K), 63 + K, 0.3)
    L = ple.Layer(hash_params(b), tb, dev_bf16(kvw), dev_bf16(cw), conv_dilation=cfg.conv_dilation, eps=cfg.eps)
    hidden = wl.make_hidden(cfg, T=max(cfg.T, 1))[:cfg.T]
    log(f"decode tail {case}: T={cfg.T} R={b.R} K={K} d={cfg.conv_dilation} hint={hint}")
    plain = _run_fused_both(cfg, b, L, hidden, with_ctx=not fresh, with_state=not fresh, max_request_tokens=0)
    tail = _run_fused_both(cfg, b, L, hidden, with_ctx=not fresh, with_state=not fresh, max_request_tokens=hint)
    for name, x, y in zip(["out", "gate", "conv input", "state out", "context out", "kv"], plain, tail):
        np.testing.assert_array_equal(y, x, err_msg=name)
    # and every output against the oracle: the whole chain, then each stage on the tail's own input
    out_t, gate_t, gated_t, st_t, ctx_t, kv_t = tail
    state_in = None if fresh else b.conv_state
    if cfg.T > 0:
        bb = dataclasses.replace(b, ngram_context=None if fresh else b.ngram_context, conv_state=state_in)
        ref = _oracle_chain(cfg, bb, table, scales, kvw, cw, hidden)
        assert np.abs(bf16_f64(out_t) - bf16_f64(ref["y"])).max() <= CONV_ABS_TOL
        _check_kv(kv_t, ref["kv"], ref["rows"], kvw)
    check_gate_conv_stages(hidden, kv_t, gate_t, gated_t, out_t, b.qsl, cw, cfg.conv_dilation, cfg.eps,
                           conv_state=state_in, state_out_gpu=None)
    # the carried conv state: the last S conv inputs of state ++ the window (the tail's own conv input)
    _, st_want = oracle.conv(gated_t if cfg.T else np.zeros((0, cfg.N), np.uint16), b.qsl, cw, cfg.conv_dilation,
                             state=state_in, want_state_out=True)
    np.testing.assert_array_equal(st_t, st_want)
    _, ctx_want = oracle.ngram_ids(b.input_ids, b.qsl, b.multipliers[0], b.vocab_sizes, b.offsets,
                                   context_len=cfg.context_len, heads_per_ngram=cfg.heads_per_ngram,
                                   eos_token_id=wl.EOS, ngram_context=None if fresh else b.ngram_context,
                                   want_context_out=True)
    np.testing.assert_array_equal(ctx_t, ctx_want)


def test_wrong_hint_keeps_short_requests_exact():
    """A max_request_tokens hint smaller than the batch's longest request gives unspecified results for
    the longer requests but stays within every buffer: the call succeeds, and requests of at most four
    tokens (the tail kernel's token slots) come out exactly as on the plain path, as does every carried
    context.  Requests of 7, 1, 13, 3, 0 and 2 tokens with the hint 2."""
    import dataclasses
    base = wl.CONFIGS[1]
    lens = [7, 1, 13, 3, 0, 2]
    rng = np.random.default_rng(91)
    cfg = dataclasses.replace(base, idx=61, T=int(sum(lens)))
    b = wl.make_batch(base, with_context=True, with_state=True)
    R = len(lens)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S = (cfg.conv_kernel - 1) * cfg.conv_dilation
    b = dataclasses.replace(b, cfg=cfg, input_ids=rng.integers(0, 1000, size=cfg.T).astype(np.int32), qsl=qsl,
                            ngram_context=rng.integers(0, 1000, size=(R, cfg.context_len)).astype(np.int32),
                            conv_state=wl.normal_bf16((R, S, cfg.N), 92, 0.125))
    table, scales, tb, keep = _table_dev(cfg)
    L = ple.Layer(hash_params(b), tb, dev_bf16(wl.make_kv_weight(cfg)), dev_bf16(wl.normal_bf16((cfg.N, 4), 93, 0.3)),
                  conv_dilation=cfg.conv_dilation, eps=cfg.eps)
    hidden = wl.make_hidden(cfg, T=cfg.T)
    log(f"wrong hint: lens={lens} hint=2")
    plain = _run_fused_both(cfg, b, L, hidden, with_ctx=True, with_state=True, max_request_tokens=0)
    hinted = _run_fused_both(cfg, b, L, hidden, with_ctx=True, with_state=True, max_request_tokens=2)
    np.testing.assert_array_equal(hinted[4], plain[4], err_msg="context out")
    checked = 0
    for r, n in enumerate(lens):
        if n > 4:
            continue
        rows = slice(qsl[r], qsl[r + 1])
        for name, i in (("out", 0), ("gate", 1), ("conv input", 2)):
            np.testing.assert_array_equal(hinted[i][rows], plain[i][rows], err_msg=f"{name}, request {r}")
        np.testing.assert_array_equal(hinted[3][r], plain[3][r], err_msg=f"state out, request {r}")
        checked += 1
    assert checked == 4


def test_prefill_with_prefetched_rows_equals_plain():
    cfg = wl.CONFIGS[2]
    b = wl.make_batch(cfg)
    L, table, scales, kvw, cw, keep = _layer(cfg, b)
    hidden = dev_bf16(wl.make_hidden(cfg))
    toks, qsl, ctx = dev(b.input_ids), dev(b.qsl), dev(b.ngram_context)
    plain = ple.ple_prefill_fused(L, toks, qsl, hidden, ngram_context=ctx)
    side = torch.cuda.Stream()
    staging = torch.empty((cfg.T, cfg.H * cfg.D), dtype=torch.bfloat16, device=DEV)
    ev0 = torch.cuda.Event()
    ev0.record()
    side.wait_event(ev0)
    ple.ple_prefetch(L, toks, qsl, staging, ngram_context=ctx, stream=side)
    ev = torch.cuda.Event()
    ev.record(side)
    torch.cuda.current_stream().wait_event(ev)
    pre = ple.ple_prefill_fused(L, toks, qsl, hidden, prefetched_rows=staging, ngram_context=ctx)
    assert torch.equal(plain, pre)


def test_prefill_empty_batch():
    cfg = wl.CONFIGS[1]
    b = wl.make_batch(cfg)
    L, *_ = _layer(cfg, b)
    out = ple.ple_prefill_fused(L, torch.zeros(0, dtype=torch.int32, device=DEV),
                                torch.zeros(1, dtype=torch.int32, device=DEV),
                                torch.zeros((0, cfg.N), dtype=torch.bfloat16, device=DEV),
                                workspace=torch.empty(256, dtype=torch.uint8, device=DEV))
    assert out.shape == (0, cfg.N)


def test_repeat_runs_bit_identical():
    cfg = wl.CONFIGS[2]
    b = wl.make_batch(cfg)
    L, *_ = _layer(cfg, b)
    hidden = dev_bf16(wl.make_hidden(cfg))
    a = ple.ple_prefill_fused(L, dev(b.input_ids), dev(b.qsl), hidden, ngram_context=dev(b.ngram_context))
    c = ple.ple_prefill_fused(L, dev(b.input_ids), dev(b.qsl), hidden, ngram_context=dev(b.ngram_context))
    assert torch.equal(a, c)


def test_host_mapped_table_matches_hbm():
    cfg = wl.CONFIGS[2]
    b = wl.make_batch(cfg)
    table, _ = wl.make_table(cfg)
    hb = ple.ple_host_alloc(table.nbytes)
    hv = hb.numpy(np.uint16, table.shape)
    hv[...] = table
    tb_host = ple.Table(hb.device, cfg.num_rows, cfg.D, ple.PLE_DTYPE_BF16)
    tb_dev = ple.Table.from_tensor(dev_bf16(table))
    hp = hash_params(b)
    r_host = ple.ple_lookup(hp, tb_host, dev(b.input_ids), dev(b.qsl), ngram_context=dev(b.ngram_context))
    r_dev = ple.ple_lookup(hp, tb_dev, dev(b.input_ids), dev(b.qsl), ngram_context=dev(b.ngram_context))
    torch.cuda.synchronize()
    assert torch.equal(r_host, r_dev)
    hb.close()


def test_cu_masked_stream_prefetch():
    cfg = wl.CONFIGS[2]
    b = wl.make_batch(cfg)
    L, *_ = _layer(cfg, b)
    s = ple.ple_stream_create_cu_masked(64)
    try:
        staging = torch.empty((cfg.T, cfg.H * cfg.D), dtype=torch.bfloat16, device=DEV)
        ev0 = torch.cuda.Event()
        ev0.record()
        s.wait_event(ev0)
        ple.ple_prefetch(L, dev(b.input_ids), dev(b.qsl), staging, ngram_context=dev(b.ngram_context), stream=s)
        s.synchronize()
        ref = ple.ple_lookup(L.hash, L.table, dev(b.input_ids), dev(b.qsl), ngram_context=dev(b.ngram_context))
        assert torch.equal(staging, ref)
    finally:
        torch.cuda.synchronize()
        ple.ple_stream_destroy(s)


# ------------------------------------------------------------------ global-scale fp8 and NVFP4 tables

def _nvfp4_dev(codes, bs, t):
    keep = (dev(codes), dev(bs), dev(np.asarray([t], dtype=np.float32)))
    return ple.Table.nvfp4(*keep), keep


def test_lookup_fp8_global_scale():
    cfg = _small_fp8_cfg()
    b = wl.make_batch(cfg)
    q, _ = wl.make_table(cfg)
    s = np.float32(0.0173)
    tb = ple.Table.from_tensor(dev(q), dev(np.asarray([s], np.float32)))
    assert tb.dtype == ple.PLE_DTYPE_FP8_E4M3_GLOBAL
    ids = oracle_ids(b)
    rows = ple.ple_lookup(hash_params(b), tb, dev(b.input_ids), dev(b.qsl))
    np.testing.assert_array_equal(host_bits(rows), oracle.gather_fp8_global(q, s, ids).reshape(cfg.T, -1))


def test_fp8_global_every_code():
    rng = np.random.default_rng(11)
    codes = np.stack([rng.permutation(256) for _ in range(32)]).astype(np.uint8)
    ids = rng.integers(0, 32, size=(40, 2)).astype(np.int32)
    for s in (np.float32(1.0), np.float32(2.0 ** -30), np.float32(7.5e28)):
        tb = ple.Table.from_tensor(dev(codes), dev(np.asarray([s], np.float32)))
        rows = ple.ple_gather(tb, dev(ids))
        np.testing.assert_array_equal(host_bits(rows), oracle.gather_fp8_global(codes, s, ids).reshape(40, -1))


def test_nvfp4_golden_cases_on_gpu():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        D = case["dim"]
        codes = np.asarray(case["codes"], dtype=np.uint8).reshape(1, D // 2)
        bs = np.asarray(case["block_scales"], dtype=np.uint8).reshape(1, D // 16)
        t = np.uint32(int(case["tensor_scale_bits"], 16)).view(np.float32)
        tb, keep = _nvfp4_dev(codes, bs, t)
        rows = ple.ple_gather(tb, dev(np.zeros((1, 1), np.int32)))
        assert host_bits(rows)[0].tolist() == [int(x, 16) for x in case["expected_bf16"]], case["name"]


@pytest.mark.parametrize("D", [32, 64, 512, 96])
def test_gather_nvfp4_every_code(D):
    rng = np.random.default_rng(D + 1)
    nrows = 500
    codes = rng.integers(0, 256, size=(nrows, D // 2), dtype=np.uint8)
    bs = rng.integers(0, 256, size=(nrows, D // 16), dtype=np.uint8)  # includes NaN and zero scales
    t = np.float32(0.031)
    ids = rng.integers(0, nrows, size=(211, 3)).astype(np.int32)
    tb, keep = _nvfp4_dev(codes, bs, t)
    rows = ple.ple_gather(tb, dev(ids))
    np.testing.assert_array_equal(host_bits(rows), oracle.gather_nvfp4(codes, bs, t, ids).reshape(211, -1))


def test_lookup_nvfp4_and_fused_prefill():
    cfg = wl.CONFIGS[1]
    b = wl.make_batch(cfg, with_context=True, with_state=True)
    codes, bs, t = wl.make_nvfp4_table(cfg.num_rows, cfg.D, cfg.seed)
    tb, keep = _nvfp4_dev(codes, bs, t)
    ids = oracle_ids(b)
    rows = ple.ple_lookup(hash_params(b), tb, dev(b.input_ids), dev(b.qsl), ngram_context=dev(b.ngram_context))
    np.testing.assert_array_equal(host_bits(rows), oracle.gather_nvfp4(codes, bs, t, ids).reshape(cfg.T, -1))
    kvw, cw, hidden = wl.make_kv_weight(cfg), wl.make_conv_weight(cfg), wl.make_hidden(cfg)
    L = ple.Layer(hash_params(b), tb, dev_bf16(kvw), dev_bf16(cw), conv_dilation=cfg.conv_dilation, eps=cfg.eps)
    out = ple.ple_prefill_fused(L, dev(b.input_ids), dev(b.qsl), dev_bf16(hidden),
                                ngram_context=dev(b.ngram_context), conv_state=dev_bf16(b.conv_state))
    ref = _oracle_chain(cfg, b, codes, (bs, t), kvw, cw, hidden)
    assert np.abs(bf16_f64(host_bits(out)) - bf16_f64(ref["y"])).max() <= CONV_ABS_TOL


# ------------------------------------------------------------------ dedup prefetch

@pytest.mark.parametrize("variant", ["cfg1", "cfg2", "cfg1-nvfp4", "repeats"])
def test_prefetch_dedup_equals_prefetch(variant):
    cfg = wl.CONFIGS[2 if variant == "cfg2" else 1]
    b = wl.make_batch(cfg, with_context=(variant != "repeats"))
    toks = b.input_ids.copy()
    if variant == "repeats":  # every token the same: only the first positions differ (EOS windows)
        toks[:] = 77
    if variant == "cfg1-nvfp4":
        codes, bs, t = wl.make_nvfp4_table(cfg.num_rows, cfg.D, cfg.seed)
        tb, keep = _nvfp4_dev(codes, bs, t)
        L = ple.Layer(hash_params(b), tb, dev_bf16(wl.make_kv_weight(cfg)), dev_bf16(wl.make_conv_weight(cfg)),
                      conv_dilation=cfg.conv_dilation, eps=cfg.eps)
    else:
        L, table, scales, kvw, cw, keep = _layer(cfg, b)
    ctx = None if b.ngram_context is None else dev(b.ngram_context)
    d_toks, d_qsl = dev(toks), dev(b.qsl)
    plain = torch.empty((cfg.T, cfg.H * cfg.D), dtype=torch.bfloat16, device=DEV)
    ple.ple_prefetch(L, d_toks, d_qsl, plain, ngram_context=ctx)
    staging = torch.full_like(plain, float("nan"))
    nu = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    ple.ple_prefetch_dedup(L, d_toks, d_qsl, staging, num_unique=nu, ngram_context=ctx)
    ids = oracle.ngram_ids(toks, b.qsl, b.multipliers[0], b.vocab_sizes, b.offsets, context_len=cfg.context_len,
                           heads_per_ngram=cfg.heads_per_ngram, eos_token_id=wl.EOS, ngram_context=b.ngram_context)
    # against the oracle's gather of the oracle's IDs, then against the plain prefetch
    if variant == "cfg1-nvfp4":
        want = oracle.gather_nvfp4(codes, bs, t, ids)
    else:
        want = oracle.gather_bf16(table, ids)
    np.testing.assert_array_equal(host_bits(staging), want.reshape(cfg.T, -1))
    assert torch.equal(staging.view(torch.int16), plain.view(torch.int16))
    assert int(nu.item()) == len(np.unique(ids))
    if variant == "repeats":
        assert int(nu.item()) < ids.size // 2


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8-global", "nvfp4"])
def test_prefetch_dedup_rows_of_512(fmt):
    """The deduplicating prefetch on 512-element rows in every table format (the list of distinct rows
    walked by the per-lane row stream, then the repeats copied) equals the oracle's gather of the
    oracle's IDs and the plain prefetch, bit for bit."""
    import dataclasses
    base = wl.CONFIGS[4] if fmt.startswith("fp8") else wl.CONFIGS[3]
    cfg = dataclasses.replace(base, idx=41, T=700, vocab_base=5003)
    b = wl.make_batch(cfg)
    if fmt == "nvfp4":
        codes, bs, t = wl.make_nvfp4_table(cfg.num_rows, cfg.D, cfg.seed)
        tb, keep = _nvfp4_dev(codes, bs, t)
        gather = lambda ids: oracle.gather_nvfp4(codes, bs, t, ids)  # noqa: E731
    elif fmt == "fp8-global":
        q, _ = wl.make_table(cfg)
        keep = (dev(q), dev(np.asarray([0.0173], np.float32)))
        tb = ple.Table.from_tensor(*keep)
        gather = lambda ids: oracle.gather_fp8_global(q, np.float32(0.0173), ids)  # noqa: E731
    else:
        q, sc, tb, keep = _table_dev(cfg)
        gather = (lambda ids: oracle.gather_bf16(q, ids)) if fmt == "bf16" else \
            (lambda ids: oracle.gather_fp8(q, sc, ids))
    L = ple.Layer(hash_params(b), tb, dev_bf16(wl.make_kv_weight(cfg)), dev_bf16(wl.make_conv_weight(cfg)),
                  conv_dilation=cfg.conv_dilation, eps=cfg.eps)
    d_toks, d_qsl = dev(b.input_ids), dev(b.qsl)
    plain = torch.empty((cfg.T, cfg.H * cfg.D), dtype=torch.bfloat16, device=DEV)
    ple.ple_prefetch(L, d_toks, d_qsl, plain)
    staging = torch.full_like(plain, float("nan"))
    nu = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    ple.ple_prefetch_dedup(L, d_toks, d_qsl, staging, num_unique=nu)
    ids = oracle_ids(b)
    np.testing.assert_array_equal(host_bits(staging), gather(ids).reshape(cfg.T, -1))
    assert torch.equal(staging.view(torch.int16), plain.view(torch.int16))
    assert int(nu.item()) == len(np.unique(ids)) < ids.size  # the Zipf batch repeats rows


def test_prefetch_dedup_plan_fetch_on_two_streams():
    """The two halves, the plan of the second layer on its own stream beside the first layer's fetch
    (each layer its own workspace, the fetch ordered after its plan by an event), equal the oracle's
    gather of each layer's oracle IDs, bit for bit, with the distinct-row counts."""
    cfg = wl.CONFIGS[1]
    b = wl.make_batch(cfg, layers=2, with_context=False)
    L0, table, scales, kvw, cw, keep = _layer(cfg, b)
    layers = [ple.Layer(hash_params(b, l), L0.table, L0.kv_weight, L0.conv_weight, conv_dilation=cfg.conv_dilation,
                        eps=cfg.eps) for l in range(2)]
    d_toks, d_qsl = dev(b.input_ids), dev(b.qsl)
    need = ple.ple_prefetch_dedup_workspace_bytes(cfg.T, cfg.H)
    ws = [torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(2)]
    staging = [torch.full((cfg.T, cfg.H * cfg.D), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    nu = torch.full((2,), -1, dtype=torch.int32, device=DEV)
    plan_s, fetch_s = torch.cuda.Stream(), torch.cuda.Stream()
    planned = [torch.cuda.Event() for _ in range(2)]
    torch.cuda.synchronize()
    ple.ple_prefetch_dedup_plan(layers[0], d_toks, d_qsl, ws[0], stream=plan_s)
    planned[0].record(plan_s)
    fetch_s.wait_event(planned[0])
    ple.ple_prefetch_dedup_fetch(layers[0], cfg.T, ws[0], staging[0], num_unique=nu[0:1], stream=fetch_s)
    ple.ple_prefetch_dedup_plan(layers[1], d_toks, d_qsl, ws[1], stream=plan_s)
    planned[1].record(plan_s)
    fetch_s.wait_event(planned[1])
    ple.ple_prefetch_dedup_fetch(layers[1], cfg.T, ws[1], staging[1], num_unique=nu[1:2], stream=fetch_s)
    torch.cuda.synchronize()
    for l in range(2):
        ids = oracle.ngram_ids(b.input_ids, b.qsl, b.multipliers[l], b.vocab_sizes, b.offsets,
                               context_len=cfg.context_len, heads_per_ngram=cfg.heads_per_ngram, eos_token_id=wl.EOS)
        np.testing.assert_array_equal(host_bits(staging[l]), oracle.gather_bf16(table, ids).reshape(cfg.T, -1))
        assert int(nu[l].item()) == len(np.unique(ids))


def test_prefetch_dedup_empty_batch_counts_zero():
    cfg = wl.CONFIGS[1]
    b = wl.make_batch(cfg)
    L, table, scales, kvw, cw, keep = _layer(cfg, b)
    nu = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    staging = torch.empty((0, cfg.H * cfg.D), dtype=torch.bfloat16, device=DEV)
    ple.ple_prefetch_dedup(L, dev(np.zeros(0, np.int32)), dev(np.zeros(1, np.int32)), staging, num_unique=nu)
    assert int(nu.item()) == 0


# ------------------------------------------------------------------ data-parallel shards (one GPU)

@pytest.mark.parametrize("E,W,counts", [(1, 8, [37]), (2, 512, [300, 123]), (4, 2048, [17, 0, 64, 5]),
                                        (3, 96, [1000, 999, 1])])
def test_select_rows_parity(E, W, counts):
    rng = np.random.default_rng(E * 100 + W)
    S = max(counts)
    gathered = rng.integers(0, 65536, size=(E, E * S, W), dtype=np.uint16)
    g = dev_bf16(gathered)
    for r in range(E):
        out = ple.ple_select_rows(g, r, counts[r])
        np.testing.assert_array_equal(host_bits(out), oracle.select_rows(gathered, r, counts[r]))


def test_sharded_lookup_equals_unsharded():
    """The whole one-GPU data flow of a table sharded over E replicas: each
    replica's batch padded into a slot, each head shard looked up over every
    slot, the shards stacked (the all-gather), and each replica's window
    selected: the same rows as the replica's own unsharded lookup."""
    cfg = wl.CONFIGS[2]
    E = 4
    b = wl.make_batch(cfg)
    table_h, _ = wl.make_table(cfg)
    tb = ple.Table.from_tensor(dev_bf16(table_h))
    # split the 256 one-token requests into E replicas of uneven sizes
    cuts = [0, 40, 130, 131, 256]
    counts = [cuts[r + 1] - cuts[r] for r in range(E)]
    slot, _ = ple.ple_dp_gather_slot(counts, E, 0)
    toks = np.full(E * slot, wl.EOS, dtype=np.int32)
    ctx = np.full((E * slot, cfg.context_len), wl.EOS, dtype=np.int32)
    for r in range(E):
        s0, off = cuts[r], ple.ple_dp_gather_slot(counts, E, r)[1]
        toks[off:off + counts[r]] = b.input_ids[s0:s0 + counts[r]]
        ctx[off:off + counts[r]] = b.ngram_context[s0:s0 + counts[r]]
    qsl = np.arange(E * slot + 1, dtype=np.int32)  # every slot position its own one-token request
    shards = []
    for k in range(E):
        first, per = ple.ple_head_shard(cfg.H, 1, 0, E, k)
        hp = hash_params(b, first_head=first, num_heads=per)
        shards.append(ple.ple_lookup(hp, tb, dev(toks), dev(qsl), ngram_context=dev(ctx)))
    gathered = torch.stack(shards)  # [E][E*slot][per*D]
    for r in range(E):
        s0 = cuts[r]
        mine = ple.ple_select_rows(gathered, r, counts[r])
        qr = np.arange(counts[r] + 1, dtype=np.int32)
        full = ple.ple_lookup(hash_params(b), tb, dev(b.input_ids[s0:s0 + counts[r]]), dev(qr),
                              ngram_context=dev(b.ngram_context[s0:s0 + counts[r]]))
        assert torch.equal(mine.view(torch.int16), full.view(torch.int16)), r


# ------------------------------------------------------------------ speculative decode commit

def _spec_hash(C, seed):
    H = 2 * C
    V = wl.primes_from(1000 + 50 * seed, H)
    off = np.concatenate([[0], np.cumsum(V)[:-1]]).astype(np.int64)
    m = wl.multipliers(seed, 1, H, C + 1)[0]
    return dict(multipliers=m, vocab_sizes=np.asarray(V, np.int64), offsets=off, context_len=C,
                heads_per_ngram=2, eos_token_id=wl.EOS)


SPEC_CASES = [
    # (R, max_window, N, K, d, C, with_state)
    (256, 4, 2048, 4, 3, 2, True),    # decode-shaped batch, 3 drafts per request
    (256, 4, 2048, 4, 3, 2, False),
    (37, 9, 64, 7, 2, 3, True),       # wider windows than the state, generic kernel size
    (5, 1, 8, 2, 1, 1, True),         # one-token windows: plain decode
    (6, 0, 16, 4, 3, 2, True),        # empty windows: state passes through
]


@pytest.mark.parametrize("case", range(len(SPEC_CASES)))
def test_spec_commit_parity(case):
    R, maxw, N, K, d, C, with_state = SPEC_CASES[case]
    log(f"spec commit case {case}: R={R} window<={maxw} N={N} K={K} d={d} C={C} state={with_state}")
    S = (K - 1) * d
    lens = wl.uniform_ints(900 + case, R, 0 if maxw == 0 else 1, maxw + 1) if maxw else np.zeros(R, np.int64)
    qsl = wl.qsl_from_lengths(lens)
    T = int(qsl[-1])
    tok = wl.uniform_ints(910 + case, T, 1, 151936).astype(np.int32)
    x = wl.normal_bf16((T, N), 920 + case, 0.5)
    # Counts cover -1 .. window+1 so both clamps are exercised.
    acc = (wl.uniform_ints(930 + case, R, 0, 1 << 20) % (lens + 3) - 1).astype(np.int32)
    st = wl.normal_bf16((R, S, N), 940 + case, 0.25) if with_state else None
    ctx = wl.uniform_ints(950 + case, R * C, 1, 151936).astype(np.int32).reshape(R, C) if with_state else None
    ha = _spec_hash(C, case)
    st_want, ctx_want = oracle.spec_commit(tok, x, qsl, acc, conv_kernel=K, dilation=d, conv_state=st,
                                           hash_args=ha, ngram_context=ctx)
    hp = ple.HashParams(ha["multipliers"], ha["vocab_sizes"], ha["offsets"], heads_per_ngram=2, context_len=C,
                        eos_token_id=wl.EOS)
    st_out = torch.full((R, S, N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ctx_out = torch.full((R, C), -7, dtype=torch.int32, device=DEV)
    xd = dev_bf16(x) if T else torch.zeros((0, N), dtype=torch.bfloat16, device=DEV)
    ple.ple_spec_commit(dev(tok) if T else torch.zeros(0, dtype=torch.int32, device=DEV), dev(qsl), dev(acc),
                        hash=hp, ngram_context=None if ctx is None else dev(ctx), ngram_context_out=ctx_out, x=xd,
                        conv_kernel=K, conv_dilation=d, conv_state=None if st is None else dev_bf16(st),
                        conv_state_out=st_out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(st_out), st_want)
    np.testing.assert_array_equal(ctx_out.cpu().numpy(), ctx_want)


def test_spec_decode_chain_matches_oracle():
    """Three verify + commit steps: ids, conv output and carried state against the oracle's chain."""
    R, N, K, d, C = 24, 64, 4, 3, 2
    S = (K - 1) * d
    ha = _spec_hash(C, 7)
    hp = ple.HashParams(ha["multipliers"], ha["vocab_sizes"], ha["offsets"], heads_per_ngram=2, context_len=C,
                        eos_token_id=wl.EOS)
    w = wl.uniform_bf16((N, K), 960, -0.5, 0.5)
    wd = dev_bf16(w)
    st_o = np.zeros((R, S, N), np.uint16)
    ctx_o = np.full((R, C), wl.EOS, np.int32)
    st_g, ctx_g = dev_bf16(st_o), dev(ctx_o)
    for step in range(3):
        lens = wl.uniform_ints(970 + step, R, 1, 5)
        qsl = wl.qsl_from_lengths(lens)
        T = int(qsl[-1])
        tok = wl.uniform_ints(980 + step, T, 1, 151936).astype(np.int32)
        x = wl.normal_bf16((T, N), 990 + step, 0.5)
        acc = (wl.uniform_ints(1000 + step, R, 0, 1 << 20) % lens + 1).astype(np.int32)
        log(f"spec chain step {step}: T={T}")
        ids_want = oracle.ngram_ids(tok, qsl, ngram_context=ctx_o, **ha)
        y_want = oracle.conv(x, qsl, w, d, state=st_o)
        st_o, ctx_o = oracle.spec_commit(tok, x, qsl, acc, conv_kernel=K, dilation=d, conv_state=st_o,
                                         hash_args=ha, ngram_context=ctx_o)
        tok_d, qsl_d, x_d = dev(tok), dev(qsl), dev_bf16(x)
        ids = ple.ple_ngram_ids(hp, tok_d, qsl_d, ngram_context=ctx_g)
        y = ple.ple_conv(x_d, qsl_d, wd, dilation=d, conv_state=st_g)
        st_n = torch.empty((R, S, N), dtype=torch.bfloat16, device=DEV)
        ctx_n = torch.empty((R, C), dtype=torch.int32, device=DEV)
        ple.ple_spec_commit(tok_d, qsl_d, dev(acc), hash=hp, ngram_context=ctx_g, ngram_context_out=ctx_n, x=x_d,
                            conv_kernel=K, conv_dilation=d, conv_state=st_g, conv_state_out=st_n)
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_want)
        got = host_bits(y)
        assert np.abs(bf16_f64(got) - bf16_f64(y_want)).max() <= CONV_ABS_TOL
        assert bf16_ulp_distance(got, y_want).max() <= 1
        np.testing.assert_array_equal(host_bits(st_n), st_o)
        np.testing.assert_array_equal(ctx_n.cpu().numpy(), ctx_o)
        st_g, ctx_g = st_n, ctx_n


def test_spec_verify_fused_then_commit():
    """Verify window through ple_prefill_fused, then commit from the conv input left in its workspace."""
    cfg = wl.CONFIGS[1]
    b = wl.make_batch(cfg, with_context=True, with_state=True)
    L, table, scales, kvw, cw, keep = _layer(cfg, b)
    hidden = wl.make_hidden(cfg)
    ref = _oracle_chain(cfg, b, table, scales, kvw, cw, hidden)
    acc = np.asarray([3, 1, 0, 3], np.int32)   # windows are 7, 1, 13, 3 tokens
    st_want, ctx_want = oracle.spec_commit(
        b.input_ids, ref["gated"], b.qsl, acc, conv_kernel=cfg.conv_kernel, dilation=cfg.conv_dilation,
        conv_state=b.conv_state, ngram_context=b.ngram_context,
        hash_args=dict(multipliers=b.multipliers[0], vocab_sizes=b.vocab_sizes, offsets=b.offsets,
                       context_len=cfg.context_len, heads_per_ngram=cfg.heads_per_ngram, eos_token_id=wl.EOS))
    T = cfg.T
    ws = torch.empty((ple.ple_prefill_workspace_bytes(L, T),), dtype=torch.uint8, device=DEV)
    toks, qsl = dev(b.input_ids), dev(b.qsl)
    ctx, st = dev(b.ngram_context), dev_bf16(b.conv_state)
    out = ple.ple_prefill_fused(L, toks, qsl, dev_bf16(hidden), ngram_context=ctx, conv_state=st, workspace=ws)
    assert np.abs(bf16_f64(host_bits(out)) - bf16_f64(ref["y"])).max() <= CONV_ABS_TOL
    x = ple.prefill_conv_input(L, ws, T)
    assert np.abs(bf16_f64(host_bits(x)) - bf16_f64(ref["gated"])).max() <= GATE_ABS_TOL
    st_out = torch.empty((b.R, cfg.S, cfg.N), dtype=torch.bfloat16, device=DEV)
    ctx_out = torch.empty((b.R, cfg.context_len), dtype=torch.int32, device=DEV)
    ple.ple_spec_commit(toks, qsl, dev(acc), hash=L.hash, ngram_context=ctx, ngram_context_out=ctx_out, x=x,
                        conv_kernel=cfg.conv_kernel, conv_dilation=cfg.conv_dilation, conv_state=st,
                        conv_state_out=st_out)
    np.testing.assert_array_equal(ctx_out.cpu().numpy(), ctx_want)
    assert np.abs(bf16_f64(host_bits(st_out)) - bf16_f64(st_want)).max() <= GATE_ABS_TOL
    # request 2 kept nothing: its state is the input state, bit for bit
    np.testing.assert_array_equal(host_bits(st_out)[2], b.conv_state[2])


def test_spec_step_graph_replay_matches_eager():
    """Verify + commit captured in a HIP graph: every replay equals the eager step, with eager work in between."""
    cfg = wl.CONFIGS[2]
    b = wl.make_batch(cfg)
    L, *_ = _layer(cfg, b)
    W, R = 2, 64
    T = R * W
    toks = dev(wl.make_tokens(cfg, T=T))
    qsl = dev(np.arange(0, T + 1, W, dtype=np.int32))
    acc = dev(wl.uniform_ints(1234, R, 0, W + 2))
    hidden = dev_bf16(wl.make_hidden(cfg, T=T))
    ctx, st = dev(b.ngram_context[:R]), dev_bf16(b.conv_state[:R])
    ws = torch.empty((ple.ple_prefill_workspace_bytes(L, T),), dtype=torch.uint8, device=DEV)
    x = ple.prefill_conv_input(L, ws, T)
    out = torch.empty((T, cfg.N), dtype=torch.bfloat16, device=DEV)
    st_out = torch.empty((R, cfg.S, cfg.N), dtype=torch.bfloat16, device=DEV)
    ctx_out = torch.empty((R, cfg.context_len), dtype=torch.int32, device=DEV)

    def step():
        ple.ple_prefill_fused(L, toks, qsl, hidden, ngram_context=ctx, conv_state=st, out=out, workspace=ws)
        ple.ple_spec_commit(toks, qsl, acc, hash=L.hash, ngram_context=ctx, ngram_context_out=ctx_out, x=x,
                            conv_kernel=cfg.conv_kernel, conv_dilation=cfg.conv_dilation, conv_state=st,
                            conv_state_out=st_out)

    step()
    torch.cuda.synchronize()
    want = [out.clone(), st_out.clone(), ctx_out.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (out, st_out, ctx_out):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"graph replay {rep}")
        for got, w in zip((out, st_out, ctx_out), want):
            assert torch.equal(got, w)
        step()  # eager work between replays
        torch.cuda.synchronize()
