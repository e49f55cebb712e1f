"""Seeded synthetic workloads for the per-layer n-gram embedding (PLE) lookup path.

This module is shared by the oracle side (tests) and the GPU side (tests, bench):
it draws inputs and holds none of the path's arithmetic.  Integer streams come
from SplitMix64 evaluated at a counter (Steele, Lea and Flood, OOPSLA 2014);
large float arrays are written by the threaded C filler in ``fill.c``.

Workload recipes (token distributions, request lengths, table sizes) follow
the five configurations of the lookup benchmark: a tiny CPU-checkable batch,
a decode batch, an 8k-token prefill, an fp8 table and a host-resident table.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from functools import lru_cache

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1
EOS = 0
QWEN_VOCAB = 151936

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libplefill.so")

# stream indices inside one configuration seed
S_TOKENS, S_LENGTHS, S_MULT, S_TABLE, S_HIDDEN, S_KVW, S_CONVW, S_CTX, S_STATE, S_PERM = range(10)


def build_filler(force: bool = True) -> str:
    """Compile fill.c into libplefill.so (gcc, no HIP)."""
    src = os.path.join(_HERE, "fill.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


@lru_cache(maxsize=1)
def _lib():
    if not os.path.exists(_LIB_PATH):
        build_filler(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, U64, D, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_int
    lib.gen_normal_bf16.argtypes = [P, I64, U64, D, I]
    lib.gen_normal_f32.argtypes = [P, I64, U64, D, I]
    lib.gen_uniform_bf16.argtypes = [P, I64, U64, D, D, I]
    lib.gen_fp8_table.argtypes = [P, P, I64, ctypes.c_int32, U64, D, I]
    lib.gen_fp8_table.restype = ctypes.c_int
    lib.gen_uniform_bytes.argtypes = [P, I64, U64, ctypes.c_int, ctypes.c_int, I]
    lib.gen_store_bf16.argtypes = [ctypes.c_float]
    lib.gen_store_bf16.restype = ctypes.c_uint16
    lib.gen_store_e4m3fn.argtypes = [ctypes.c_float]
    lib.gen_store_e4m3fn.restype = ctypes.c_uint8
    return lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# integer streams
# ----------------------------------------------------------------------------

def stream_seed(config_seed: int, stream: int) -> int:
    return (config_seed + GAMMA * stream) & MASK64


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Values start..start+n-1 of the SplitMix64 stream that starts at `seed`."""
    with np.errstate(over="ignore"):
        i = np.arange(start, start + n, dtype=np.uint64) + np.uint64(1)
        z = np.uint64(seed) + i * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def uniform01(seed: int, n: int) -> np.ndarray:
    return (splitmix64(seed, n) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def uniform_ints(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers in [lo, hi) by multiply-shift of the top 32 bits."""
    span = hi - lo
    assert 0 < span < (1 << 32)
    top = splitmix64(seed, n) >> np.uint64(32)
    return (lo + ((top * np.uint64(span)) >> np.uint64(32)).astype(np.int64)).astype(np.int32)


def _is_prime(x: int) -> bool:
    if x < 2:
        return False
    if x % 2 == 0:
        return x == 2
    return all(x % p for p in range(3, math.isqrt(x) + 1, 2))


def primes_from(base: int, count: int) -> list[int]:
    """The `count` consecutive primes >= base (trial division)."""
    out, x = [], base
    while len(out) < count:
        if _is_prime(x):
            out.append(x)
        x += 1
    return out


def multipliers(seed: int, layers: int, heads: int, width: int) -> np.ndarray:
    """Odd int64 hash multipliers m[layer, head, j], SplitMix64 over (l, h, j) row-major."""
    z = splitmix64(seed, layers * heads * width) | np.uint64(1)
    return z.view(np.int64).reshape(layers, heads, width).copy()


def zipf_tokens(seed: int, perm_seed: int, n: int, vocab: int = QWEN_VOCAB, s: float = 1.1) -> np.ndarray:
    """Truncated Zipf(s) over ranks 1..vocab by inverse CDF; token = perm(rank-1)."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = uniform01(seed, n)
    rank0 = np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1)
    perm = np.argsort(splitmix64(perm_seed, vocab), kind="stable").astype(np.int32)
    return perm[rank0].astype(np.int32)


def geometric_lengths(seed: int, total: int, p: float = 1.0 / 512, lo: int = 1, hi: int = 4096) -> np.ndarray:
    """Request lengths ~ geometric(p) on {1,2,...}, clipped to [lo, hi], drawn until
    they cover `total` tokens; the last one is cut so the sum is exactly `total`."""
    lens, acc, start = [], 0, 0
    while acc < total:
        u = splitmix_uniform_block(seed, start)
        for x in u:
            v = 1.0 - x  # in (0, 1]
            L = 1 + int(np.floor(np.log(v) / np.log1p(-p)))
            L = min(max(L, lo), hi)
            L = min(L, total - acc)
            lens.append(L)
            acc += L
            if acc >= total:
                break
        start += 4096
    return np.asarray(lens, dtype=np.int32)


def splitmix_uniform_block(seed: int, start: int, n: int = 4096) -> np.ndarray:
    return (splitmix64(seed, n, start) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def qsl_from_lengths(lengths) -> np.ndarray:
    q = np.zeros(len(lengths) + 1, dtype=np.int32)
    q[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return q


# ----------------------------------------------------------------------------
# float fills (C filler; values depend only on (seed, index))
# ----------------------------------------------------------------------------

def _ptr(a) -> int:
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    return int(a.data_ptr())  # torch tensor (host)


def fill_normal_bf16(out, seed: int, sigma: float, threads: int | None = None):
    """Fill a uint16 (bf16 bits) host array with bf16(sigma * N(0,1))."""
    n = out.size if isinstance(out, np.ndarray) else out.numel()
    _lib().gen_normal_bf16(_ptr(out), n, seed, sigma, threads or default_threads())
    return out


def fill_normal_f32(out, seed: int, sigma: float, threads: int | None = None):
    n = out.size if isinstance(out, np.ndarray) else out.numel()
    _lib().gen_normal_f32(_ptr(out), n, seed, sigma, threads or default_threads())
    return out


def fill_uniform_bf16(out, seed: int, lo: float, hi: float, threads: int | None = None):
    n = out.size if isinstance(out, np.ndarray) else out.numel()
    _lib().gen_uniform_bf16(_ptr(out), n, seed, lo, hi, threads or default_threads())
    return out


def fill_fp8_table(q, scale, rows: int, dim: int, seed: int, sigma: float, threads: int | None = None):
    rc = _lib().gen_fp8_table(_ptr(q), _ptr(scale), rows, dim, seed, sigma, threads or default_threads())
    if rc:
        raise ValueError("fp8 table dim out of range")
    return q, scale


def normal_bf16(shape, seed: int, sigma: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    return fill_normal_bf16(out, seed, sigma)


def uniform_bf16(shape, seed: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    return fill_uniform_bf16(out, seed, lo, hi)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Config:
    idx: int
    name: str
    T: int
    heads_per_ngram: int
    context_len: int          # C: orders 2..C+1
    vocab_base: int           # head vocab sizes are the H consecutive primes >= this
    D: int
    table_dtype: str          # "bf16" | "fp8"
    N: int                    # hidden size; kv_proj maps H*D -> 2N
    conv_kernel: int
    conv_dilation: int
    tokens: str               # "uniform1000" | "uniform" | "zipf"
    requests: str             # "fixed" | "decode" | "geometric"
    with_context: bool
    with_state: bool
    host_table: bool = False
    fixed_lengths: tuple = ()
    eps: float = 1e-6

    @property
    def H(self) -> int:
        return self.context_len * self.heads_per_ngram

    @property
    def S(self) -> int:
        return (self.conv_kernel - 1) * self.conv_dilation

    @property
    def seed(self) -> int:
        return 1000 + self.idx

    @property
    def vocab_sizes(self) -> list[int]:
        return primes_from(self.vocab_base, self.H)

    @property
    def offsets(self) -> list[int]:
        v = self.vocab_sizes
        return [sum(v[:h]) for h in range(len(v))]

    @property
    def num_rows(self) -> int:
        return sum(self.vocab_sizes)


CONFIGS = {
    1: Config(1, "tiny-ragged-4req", 24, 2, 2, 9973, 32, "bf16", 128, 4, 2,
              "uniform1000", "fixed", False, False, fixed_lengths=(7, 1, 13, 3)),
    2: Config(2, "decode-256req", 256, 4, 2, 1 << 17, 256, "bf16", 2048, 4, 3,
              "uniform", "decode", True, True),
    3: Config(3, "prefill-8k-bf16-hbm", 8192, 4, 2, 1 << 20, 512, "bf16", 4096, 4, 3,
              "zipf", "geometric", False, False),
    4: Config(4, "prefill-16k-fp8-hbm", 16384, 8, 2, 1 << 21, 512, "fp8", 4096, 4, 3,
              "zipf", "geometric", False, False),
    5: Config(5, "prefill-8k-bf16-host", 8192, 4, 2, 1 << 23, 512, "bf16", 4096, 4, 3,
              "zipf", "geometric", False, False, host_table=True),
}


def make_tokens(cfg: Config, seed: int | None = None, T: int | None = None) -> np.ndarray:
    s = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    if cfg.tokens == "uniform1000":
        return uniform_ints(stream_seed(s, S_TOKENS), T, 0, 1000)
    if cfg.tokens == "uniform":
        return uniform_ints(stream_seed(s, S_TOKENS), T, 0, QWEN_VOCAB)
    return zipf_tokens(stream_seed(s, S_TOKENS), stream_seed(s, S_PERM), T)


def make_lengths(cfg: Config, seed: int | None = None, T: int | None = None) -> np.ndarray:
    s = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    if cfg.requests == "fixed":
        assert sum(cfg.fixed_lengths) == T
        return np.asarray(cfg.fixed_lengths, dtype=np.int32)
    if cfg.requests == "decode":
        return np.ones(T, dtype=np.int32)
    return geometric_lengths(stream_seed(s, S_LENGTHS), T)


@dataclasses.dataclass
class Batch:
    """Host-side (numpy) batch and per-layer parameters of one configuration."""
    cfg: Config
    input_ids: np.ndarray        # int32 [T]
    qsl: np.ndarray              # int32 [R+1]
    multipliers: np.ndarray      # int64 [L, H, C+1]
    vocab_sizes: np.ndarray      # int64 [H]
    offsets: np.ndarray          # int64 [H]
    ngram_context: np.ndarray | None   # int32 [R, C]
    conv_state: np.ndarray | None      # bf16 bits [R, S, N]

    @property
    def R(self) -> int:
        return len(self.qsl) - 1


def make_batch(cfg: Config, layers: int = 1, seed: int | None = None,
               with_context: bool | None = None, with_state: bool | None = None) -> Batch:
    s = cfg.seed if seed is None else seed
    toks = make_tokens(cfg, s)
    lens = make_lengths(cfg, s)
    qsl = qsl_from_lengths(lens)
    R = len(lens)
    mult = multipliers(stream_seed(s, S_MULT), layers, cfg.H, cfg.context_len + 1)
    wc = cfg.with_context if with_context is None else with_context
    ws = cfg.with_state if with_state is None else with_state
    ctx = None
    if wc:
        lo_hi = (0, 1000) if cfg.tokens == "uniform1000" else (0, QWEN_VOCAB)
        ctx = uniform_ints(stream_seed(s, S_CTX), R * cfg.context_len, *lo_hi).reshape(R, cfg.context_len)
    st = None
    if ws:
        st = normal_bf16((R, cfg.S, cfg.N), stream_seed(s, S_STATE), 0.125)
    return Batch(cfg, toks, qsl, mult,
                 np.asarray(cfg.vocab_sizes, dtype=np.int64),
                 np.asarray(cfg.offsets, dtype=np.int64), ctx, st)


def kv_weight_sigma(cfg: Config) -> float:
    """Projection weight scale giving key/value entries of RMS ~0.25 for
    table entries of RMS 0.02: sigma_w = 0.25 / (0.02 * sqrt(H*D))."""
    return 12.5 / float(np.sqrt(cfg.H * cfg.D))


TABLE_SIGMA = 0.02


def fill_table(cfg: Config, out_rows, out_scales=None, seed: int | None = None, threads=None):
    """Write the configuration's table into caller buffers (numpy or host torch):
    bf16 -> uint16 [rows, D]; fp8 -> uint8 [rows, D] codes + float32 [rows] scales."""
    s = stream_seed(cfg.seed if seed is None else seed, S_TABLE)
    if cfg.table_dtype == "bf16":
        fill_normal_bf16(out_rows, s, TABLE_SIGMA, threads)
    else:
        fill_fp8_table(out_rows, out_scales, cfg.num_rows, cfg.D, s, TABLE_SIGMA, threads)


def make_table(cfg: Config, seed: int | None = None):
    if cfg.table_dtype == "bf16":
        t = np.empty((cfg.num_rows, cfg.D), dtype=np.uint16)
        fill_table(cfg, t, seed=seed)
        return t, None
    q = np.empty((cfg.num_rows, cfg.D), dtype=np.uint8)
    sc = np.empty((cfg.num_rows,), dtype=np.float32)
    fill_table(cfg, q, sc, seed=seed)
    return q, sc


def uniform_bytes(shape, seed: int, lo: int, hi: int, threads=None) -> np.ndarray:
    """uint8 array, each entry uniform over the integers lo..hi (SplitMix64 at the entry's index)."""
    out = np.empty(shape, dtype=np.uint8)
    _lib().gen_uniform_bytes(out.ctypes.data, out.size, seed & MASK64, lo, hi, threads or default_threads())
    return out


# NVFP4 table recipe (no page fixes one): every byte of codes uniform over
# 0..255 (so both nibbles cover all 16 e2m1 codes), block-scale codes uniform
# over the e4m3fn codes 0x28..0x48 (0.25 .. 4), and a table scale of 0.005,
# which puts typical |values| near the bf16 table's 0.02.
NVFP4_BLOCK_SCALE_CODES = (0x28, 0x48)
NVFP4_TENSOR_SCALE = np.float32(0.005)
S_NVFP4_CODES, S_NVFP4_SCALES = 101, 102


def make_nvfp4_table(num_rows: int, dim: int, seed: int):
    """(codes uint8 [rows, D/2], block scales uint8 [rows, D/16], tensor scale float32)."""
    codes = uniform_bytes((num_rows, dim // 2), stream_seed(seed, S_NVFP4_CODES), 0, 255)
    bs = uniform_bytes((num_rows, dim // 16), stream_seed(seed, S_NVFP4_SCALES), *NVFP4_BLOCK_SCALE_CODES)
    return codes, bs, NVFP4_TENSOR_SCALE


def make_hidden(cfg: Config, seed: int | None = None, T: int | None = None) -> np.ndarray:
    T = cfg.T if T is None else T
    return normal_bf16((T, cfg.N), stream_seed(cfg.seed if seed is None else seed, S_HIDDEN), 1.0)


def make_kv_weight(cfg: Config, seed: int | None = None, layer: int = 0) -> np.ndarray:
    s = stream_seed(cfg.seed if seed is None else seed, S_KVW) + layer
    return normal_bf16((2 * cfg.N, cfg.H * cfg.D), s & MASK64, kv_weight_sigma(cfg))


def make_conv_weight(cfg: Config, seed: int | None = None) -> np.ndarray:
    return uniform_bf16((cfg.N, cfg.conv_kernel), stream_seed(cfg.seed if seed is None else seed, S_CONVW),
                        -0.5, 0.5)
