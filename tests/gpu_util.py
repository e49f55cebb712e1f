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
