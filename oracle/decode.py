"""One decode step of one layer on the host model: gather every sequence's
blocks by its table into contiguous keys/values, widen to float64 and apply
dense attention.

Sources:
  * "vLLM PagedAttention and continuous batching", "PagedAttention: fixed
    blocks, non-contiguous physical memory" and "The kernel page, and what the
    2023 runs measured": one query token per sequence reads that sequence's
    blocks through its block table; the formula is unchanged by paging.
  * "PagedAttention and Online Inference", verification plan item 1: check
    outputs against a contiguous-K/V baseline -- this module is that baseline.

Reading taken: a sequence's context length n counts the token written by this
step, so the query attends to positions 0..n-1.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import dense_attention
from .cache_ops import HostPool, gather
from .dtypes import bits_to_f64


def decode_one(pool: HostPool, layer: int, q_bits: np.ndarray, table: Sequence[int],
               n: int, scale: float, dtype: str) -> np.ndarray:
    """q_bits: [Hq][d] storage bits -> out [Hq][d] float64."""
    Kc, Vc = gather(pool, layer, table, int(n))
    return dense_attention(bits_to_f64(q_bits, dtype), bits_to_f64(Kc, dtype),
                           bits_to_f64(Vc, dtype), float(scale))


def decode_layer(pool: HostPool, layer: int, q_bits: np.ndarray, tables: Sequence[Sequence[int]],
                 lengths: Sequence[int], scale: float, dtype: str) -> np.ndarray:
    """q_bits: [S][Hq][d] -> out [S][Hq][d] float64."""
    S, Hq, d = q_bits.shape
    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        out[s] = decode_one(pool, layer, q_bits[s], tables[s], int(lengths[s]), scale, dtype)
    return out


def multi_query_one(pool: HostPool, layer: int, q_bits: np.ndarray, table: Sequence[int],
                    n: int, scale: float, dtype: str) -> np.ndarray:
    """Several new tokens of one sequence at its last positions: q_bits
    [nq][Hq][d] -> out [nq][Hq][d] float64.  Query t sits at position
    n - nq + t and attends to positions 0 .. n - nq + t.

    Sources: "vLLM PagedAttention and continuous batching", "Chunked prefill"
    (a split prefill: each chunk of a prompt attends to what the cache holds
    so far plus its own earlier tokens); "PagedAttention and Online
    Inference", section 5 (speculative decoding creates several positions at
    once).  Reading taken: the sequence's context length n counts all nq new
    tokens, already written to the cache, and the mask is causal among them.
    """
    nq = int(q_bits.shape[0])
    n = int(n)
    if nq > n:
        raise ValueError("more queries than context positions")
    Kc, Vc = gather(pool, layer, table, n)
    K, V = bits_to_f64(Kc, dtype), bits_to_f64(Vc, dtype)
    out = np.zeros(q_bits.shape, dtype=np.float64)
    for t in range(nq):
        lim = n - nq + t + 1
        out[t] = dense_attention(bits_to_f64(q_bits[t], dtype), K[:lim], V[:lim], float(scale))
    return out
