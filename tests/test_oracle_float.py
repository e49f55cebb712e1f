"""Pins for the oracle's floating-point stages (CPU only).

* FP8 decode: all 256 OCP e4m3fn codes against torch.float8_e4m3fn and the
  format's defining values ("Support PLE-Offload for Qwen3.8-Flash-Next -
  #53899", report on float8_e4m3fn PLE tables).
* bf16 rounding: exact rational rounding (fractions) on edge cases and torch's
  float32 -> bfloat16 conversion on random values.
* kv_proj: torch float64 matmul ("PR #54517 ...", 实现拆解 item 1, merged kv_proj).
* gate: closed forms (orthogonal h, k gives 1/2; v = 0 gives 0; h = k).
* conv: torch conv1d with dilation per request, Kc = 1, impulse response,
  chunked == whole with carried state ("PR #54517 ...", 实现拆解 item 2).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def bf16_bits_of_f64_rne(x: np.ndarray) -> np.ndarray:
    """Independent vectorised float64 -> bf16 round-to-nearest-even for values in
    the normal bf16 range: rounds the float64 bit pattern at 8 significant bits."""
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64).copy()
    drop = np.uint64(45)  # 52 - 7 stored mantissa bits
    lsb = (u >> drop) & np.uint64(1)
    u = u + (np.uint64((1 << 44) - 1) + lsb)
    u &= ~np.uint64((1 << 45) - 1)
    f = u.view(np.float64).astype(np.float32)  # exact
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(np.asarray(b, dtype=np.uint16)).astype(np.float64)


# ---------------------------------------------------------------- fp8 decode

def test_e4m3fn_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.e4m3fn_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
    assert np.isnan(oracle.e4m3fn_value(0x7F)) and np.isnan(oracle.e4m3fn_value(0xFF))


def test_e4m3fn_defining_values():
    assert oracle.e4m3fn_value(0x7E) == 448.0          # largest finite
    assert oracle.e4m3fn_value(0xFE) == -448.0
    assert oracle.e4m3fn_value(0x38) == 1.0            # exponent field 7 = bias
    assert oracle.e4m3fn_value(0x08) == 2.0 ** -6      # smallest normal
    assert oracle.e4m3fn_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert oracle.e4m3fn_value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert oracle.e4m3fn_value(0x77) == 240.0          # 1.875 * 2^7
    z = oracle.e4m3fn_value(0x80)
    assert z == 0.0 and np.signbit(z)


# ---------------------------------------------------------------- bf16 rounding

def _exact_bf16(x: float) -> int:
    """Nearest bf16 to x by exhaustive neighbour search in exact rationals."""
    f = np.float32(x)
    base = int(np.asarray([f], np.float32).view(np.uint32)[0] >> 16)
    X = Fraction(x)
    best = None
    for cand in (base - 1, base, base + 1, base + 2):
        if not 0 <= cand < 0x7F80 and not 0x8000 <= cand < 0xFF80:
            continue
        v = Fraction(oracle.bf16_value(cand))
        d = abs(v - X)
        key = (d, cand & 1)  # ties -> even mantissa
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_bf16_rounding_edge_cases():
    one = 1.0
    ulp = 2.0 ** -7
    cases = [one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2.0 ** -40, one + ulp / 2 - 2.0 ** -40,
             -(one + ulp / 2), 3.0e38, 1e-39, 2.0 ** -133, 2.0 ** -134 * 3, 0.1, -0.3, 123.456, 2.0 ** -126]
    for x in cases:
        assert oracle.bf16_from_double(x) == _exact_bf16(x), x
    assert oracle.bf16_from_double(float("nan")) == 0x7FC0
    assert oracle.bf16_from_double(float("inf")) == 0x7F80
    assert oracle.bf16_from_double(-float("inf")) == 0xFF80
    assert oracle.bf16_from_double(3.4e38) == 0x7F80   # rounds past the largest finite
    assert oracle.bf16_from_double(-0.0) == 0x8000


def test_bf16_rounding_vs_torch_float32():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.asarray([oracle.bf16_from_double(float(v)) for v in x], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_bf16_double_rounding_is_single():
    # values between two bf16 numbers that a float32 detour would round to a tie
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30   # just above the midpoint of 1 and 1+2^-7
    assert oracle.bf16_from_double(x) == _exact_bf16(x) == 0x3F81


# ---------------------------------------------------------------- gathers

def test_gather_fp8_vs_torch():
    rng = np.random.default_rng(1)
    rows, D = 300, 48
    codes = rng.integers(0, 256, size=(rows, D), dtype=np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scales = np.exp(rng.uniform(-12, 2, rows)).astype(np.float32)
    ids = rng.integers(0, rows, size=97).astype(np.int32)
    got = oracle.gather_fp8(codes, scales, ids)
    f = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    prod = f * torch.from_numpy(scales)[:, None]                     # one fp32 multiply
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[ids]
    np.testing.assert_array_equal(got, ref)


def test_gather_fp8_nan_codes():
    codes = np.asarray([[0x7F, 0xFF, 0x00, 0x80]], dtype=np.uint8)
    got = oracle.gather_fp8(codes, np.asarray([2.0], np.float32), np.asarray([0], np.int32))
    assert got.tolist() == [[0x7FC0, 0x7FC0, 0x0000, 0x8000]]


def test_gather_bf16_is_fancy_indexing():
    rng = np.random.default_rng(2)
    table = rng.integers(0, 65536, size=(1000, 40), dtype=np.uint16)
    ids = rng.integers(0, 1000, size=(33, 3)).astype(np.int32)
    np.testing.assert_array_equal(oracle.gather_bf16(table, ids), table[ids.reshape(-1)])


# ---------------------------------------------------------------- kv_proj

def test_kv_proj_vs_torch_matmul():
    rng = np.random.default_rng(3)
    T, K, O = 37, 96, 70
    x = wl.normal_bf16((T, K), 11, 0.02)
    w = wl.normal_bf16((O, K), 12, 12.5 / np.sqrt(K))
    got = oracle.kv_proj(x, w)
    ref64 = torch.from_numpy(bf16_to_f64(x)) @ torch.from_numpy(bf16_to_f64(w)).T
    np.testing.assert_array_equal(got, bf16_bits_of_f64_rne(ref64.numpy()))
    assert rng is not None


# ---------------------------------------------------------------- gate

def _bf(vals):
    return np.asarray([oracle.bf16_from_double(float(v)) for v in np.ravel(vals)], np.uint16).reshape(
        np.shape(vals))


def test_gate_orthogonal_is_half():
    N = 64
    h = np.zeros((1, N))
    k = np.zeros((1, N))
    h[0, 0::2] = 1.0
    k[0, 1::2] = 0.5
    v = np.linspace(-1.5, 1.5, N)[None, :]
    kv = np.concatenate([_bf(k), _bf(v)], axis=1)
    out, g = oracle.gate(_bf(h), kv)
    assert g[0] == 0.5
    np.testing.assert_array_equal(bf16_to_f64(out), bf16_to_f64(_bf(v)) / 2)  # halving is exact


def test_gate_zero_value():
    N = 32
    rng = np.random.default_rng(4)
    h = _bf(rng.standard_normal((3, N)))
    kv = np.concatenate([_bf(rng.standard_normal((3, N)) * 0.25), np.zeros((3, N), np.uint16)], axis=1)
    out, g = oracle.gate(h, kv)
    assert (out == 0).all() and ((g > 0) & (g < 1)).all()


def test_gate_h_equals_k_closed_form():
    rng = np.random.default_rng(5)
    N, eps = 256, 1e-6
    h = _bf(rng.standard_normal((4, N)) * 0.3)
    v = _bf(rng.standard_normal((4, N)))
    out, g = oracle.gate(h, np.concatenate([h, v], axis=1), eps)
    hv = bf16_to_f64(h)
    ms = (hv * hv).mean(axis=1)
    s = np.sqrt(N) * ms / (ms + eps)
    np.testing.assert_allclose(g, 1.0 / (1.0 + np.exp(-s)), rtol=1e-13)
    assert (g > 0.5).all()


def test_gate_sign_flip_symmetry():
    # g(h, -k) = 1 - g(h, k)
    rng = np.random.default_rng(6)
    N = 128
    h = _bf(rng.standard_normal((5, N)))
    k = _bf(rng.standard_normal((5, N)) * 0.25)
    v = _bf(rng.standard_normal((5, N)) * 0.25)
    _, g1 = oracle.gate(h, np.concatenate([k, v], 1))
    _, g2 = oracle.gate(h, np.concatenate([k ^ np.uint16(0x8000), v], 1))
    np.testing.assert_allclose(g1 + g2, 1.0, rtol=0, atol=1e-14)


def test_gate_range_on_config_distribution():
    cfg = wl.CONFIGS[2]
    h = wl.make_hidden(cfg)[:64]
    kv = wl.normal_bf16((64, 2 * cfg.N), 77, 0.25)
    _, g = oracle.gate(h, kv)
    assert ((g > 0) & (g < 1)).all()


# ---------------------------------------------------------------- conv

def _conv_torch_ref(x_bits, qsl, w_bits, d):
    x = torch.from_numpy(bf16_to_f64(x_bits))
    w = torch.from_numpy(bf16_to_f64(w_bits))
    N, K = w.shape
    outs = []
    for r in range(len(qsl) - 1):
        seg = x[qsl[r]:qsl[r + 1]].T[None]  # [1, N, L]
        if seg.shape[-1] == 0:
            continue
        y = torch.nn.functional.conv1d(seg, w[:, None, :], padding=(K - 1) * d, dilation=d, groups=N)
        outs.append(y[0, :, : seg.shape[-1]].T)
    return bf16_bits_of_f64_rne(torch.cat(outs).numpy())


@pytest.mark.parametrize("K,d", [(4, 1), (4, 3), (3, 2), (1, 1), (2, 5)])
def test_conv_vs_torch_conv1d(K, d):
    N = 24
    qsl = wl.qsl_from_lengths([5, 0, 17, 1, 9])
    x = wl.normal_bf16((int(qsl[-1]), N), 21, 0.7)
    w = wl.uniform_bf16((N, K), 22, -0.5, 0.5)
    np.testing.assert_array_equal(oracle.conv(x, qsl, w, d), _conv_torch_ref(x, qsl, w, d))


def test_conv_kernel1_is_elementwise():
    N = 16
    qsl = wl.qsl_from_lengths([6, 4])
    x = wl.normal_bf16((10, N), 31, 1.0)
    w = wl.uniform_bf16((N, 1), 32, -0.5, 0.5)
    want = bf16_bits_of_f64_rne(bf16_to_f64(x) * bf16_to_f64(w)[:, 0][None, :])
    np.testing.assert_array_equal(oracle.conv(x, qsl, w, 3), want)


def test_conv_impulse_response():
    N, K, d = 8, 4, 3
    x = np.zeros((20, N), np.uint16)
    x[2] = _bf(np.full(N, 1.0))
    w = wl.uniform_bf16((N, K), 33, -0.5, 0.5)
    y = oracle.conv(x, [0, 20], w, d)
    for t in range(20):
        i, rem = divmod(t - 2, d)
        if t >= 2 and rem == 0 and i < K:
            np.testing.assert_array_equal(y[t], w[:, K - 1 - i])
        else:
            assert (bf16_to_f64(y[t]) == 0).all()


def test_conv_chunked_equals_whole_with_state():
    N, K, d = 12, 4, 3
    x = wl.normal_bf16((30, N), 41, 1.0)
    w = wl.uniform_bf16((N, K), 42, -0.5, 0.5)
    whole, st_whole = oracle.conv(x, [0, 30], w, d, want_state_out=True)
    pieces, st = [], None
    for lo, hi in [(0, 4), (4, 5), (5, 19), (19, 20), (20, 30)]:
        y, st = oracle.conv(x[lo:hi], [0, hi - lo], w, d, state=st, want_state_out=True)
        pieces.append(y)
    np.testing.assert_array_equal(np.concatenate(pieces), whole)
    np.testing.assert_array_equal(st, st_whole)
    np.testing.assert_array_equal(st_whole[0], x[30 - 9:])


def test_conv_state_out_for_short_and_empty_requests():
    N, K, d = 4, 3, 2  # S = 4
    st_in = wl.normal_bf16((3, 4, N), 51, 1.0)
    x = wl.normal_bf16((3, N), 52, 1.0)
    w = wl.uniform_bf16((N, K), 53, -0.5, 0.5)
    _, so = oracle.conv(x, [0, 0, 2, 3], w, d, state=st_in, want_state_out=True)
    np.testing.assert_array_equal(so[0], st_in[0])                       # empty: unchanged
    np.testing.assert_array_equal(so[1], np.concatenate([st_in[1][2:], x[0:2]]))
    np.testing.assert_array_equal(so[2], np.concatenate([st_in[2][1:], x[2:3]]))


def _float_neighbours(x: float, n: int):
    f = np.float32(x)
    out = [f]
    up = dn = f
    for _ in range(n):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return out


def test_gather_fp8_multiply_rounds_in_fp32_first():
    # A product just below a bf16 midpoint whose fp32 rounding lands on the midpoint:
    # one fp32 multiply then RNE gives the even (upper) bf16, direct rounding the lower.
    v = Fraction(9, 8)                       # code 0x39 = 1.125
    mid = Fraction(1) + Fraction(3, 256)     # midpoint of bf16 0x3F81 and 0x3F82
    found = None
    for s in _float_neighbours(float(mid / v), 64):
        exact = v * Fraction(float(s))
        if exact < mid and Fraction(float(np.float32(9 / 8) * s)) == mid:
            found = s
            break
    assert found is not None
    got = oracle.gather_fp8(np.asarray([[0x39]], np.uint8), np.asarray([found], np.float32),
                            np.asarray([0], np.int32))
    assert got[0, 0] == 0x3F82


# ---------------------------------------------------------------- global-scale fp8 and NVFP4

def test_gather_fp8_global_vs_torch():
    """One scale for the table: torch's float8_e4m3fn decode, one fp32 multiply, bf16."""
    rng = np.random.default_rng(7)
    rows, D = 200, 64
    codes = rng.integers(0, 256, size=(rows, D), dtype=np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    ids = rng.integers(0, rows, size=77).astype(np.int32)
    for scale in (np.float32(0.0123), np.float32(3.5), np.float32(2.0 ** -20)):
        got = oracle.gather_fp8_global(codes, scale, ids)
        f = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
        ref = (f * torch.tensor(scale)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[ids]
        np.testing.assert_array_equal(got, ref)


def test_gather_fp8_global_equals_per_row_with_equal_scales():
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 256, size=(50, 32), dtype=np.uint8)
    ids = rng.integers(0, 50, size=40).astype(np.int32)
    s = np.float32(0.37)
    np.testing.assert_array_equal(oracle.gather_fp8_global(codes, s, ids),
                                  oracle.gather_fp8(codes, np.full(50, s, np.float32), ids))


def _nvfp4_golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_cases.json")) as f:
        return json.load(f)


def test_e2m1_values_match_the_format():
    want = _nvfp4_golden()["e2m1_values"]
    got = [oracle.e2m1_value(c) for c in range(16)]
    assert got == want
    assert [np.signbit(v) for v in got] == [c >= 8 for c in range(16)]


@pytest.mark.parametrize("case", _nvfp4_golden()["cases"], ids=lambda c: c["name"])
def test_gather_nvfp4_golden(case):
    D = case["dim"]
    codes = np.asarray(case["codes"], dtype=np.uint8).reshape(1, D // 2)
    bs = np.asarray(case["block_scales"], dtype=np.uint8).reshape(1, D // 16)
    t = np.uint32(int(case["tensor_scale_bits"], 16)).view(np.float32)
    got = oracle.gather_nvfp4(codes, bs, t, np.asarray([0], np.int32))[0]
    want = [int(x, 16) for x in case["expected_bf16"]]
    assert got.tolist() == want


def test_gather_nvfp4_unit_code_reduces_to_global_fp8():
    """e2m1 code 2 is exactly 1.0, so each element is e4m3fn(block scale) times the
    table scale: the global-scale fp8 gather (pinned against torch) on the block codes."""
    rng = np.random.default_rng(9)
    rows, D = 64, 64
    bs = rng.integers(0, 256, size=(rows, D // 16), dtype=np.uint8)
    codes = np.full((rows, D // 2), 0x22, dtype=np.uint8)
    ids = rng.integers(0, rows, size=30).astype(np.int32)
    t = np.float32(0.0731)
    got = oracle.gather_nvfp4(codes, bs, t, ids)
    want = oracle.gather_fp8_global(np.repeat(bs, 16, axis=1), t, ids)
    np.testing.assert_array_equal(got, want)


def test_gather_nvfp4_unit_scales_give_the_code_values():
    rng = np.random.default_rng(10)
    codes = rng.integers(0, 256, size=(10, 16), dtype=np.uint8)
    bs = np.full((10, 2), 0x38, dtype=np.uint8)  # e4m3fn 1.0
    got = oracle.gather_nvfp4(codes, bs, np.float32(1.0), np.arange(10, dtype=np.int32))
    e2m1 = _nvfp4_golden()["e2m1_values"]
    for r in range(10):
        for c in range(32):
            byte = int(codes[r, c // 2])
            v = e2m1[byte & 15] if c % 2 == 0 else e2m1[byte >> 4]
            assert oracle.bf16_value(int(got[r, c])) == v
            assert np.signbit(oracle.bf16_value(int(got[r, c]))) == np.signbit(v)
