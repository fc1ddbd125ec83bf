"""CPU oracle for the naive (expanded) form of MLA attention, stage by stage.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the tests, the smoke check in __graft_entry__ and the cpu_baseline leg of bench.py
use it.  It shares no code with the HIP library.

Page "Module 05 -- MLA: Compressing Per-Token History", section 5 (prefill and decode may want
different algebra): the NAIVE form expands k_{j,h} = U_h^K c_j and v_{j,h} = U_h^V c_j for every
cached token (section 1) and runs ordinary multi-head attention on them, each query seeing only
j <= t (section 4).  `mla_oracle.mla_reference` is this form end to end; the two stages are split
out here so that a GPU expansion and a GPU attention over expanded keys and values can each be
checked on their own (the attention against the GPU's own rounded keys and values).

Reading taken where the pages are silent: a GPU naive form stores the
expanded keys and values as bf16, rounded to nearest even, like the cache they come from.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import bf16_bits_to_f64, expand_keys, expand_values, softmax_attention


def expanded_kv(cache_bits_b: np.ndarray, w_k_bits: np.ndarray, w_v_bits: np.ndarray, n: int):
    """Keys and values of positions 0 .. n-1 of one sequence, every head, float64.
    cache_bits_b [L, R], w_*_bits [H, D, R] -> (k [n, H, D], v [n, H, D])."""
    c = bf16_bits_to_f64(cache_bits_b[:n])
    H, D, _ = w_k_bits.shape
    k = np.empty((n, H, D))
    v = np.empty((n, H, D))
    for h in range(H):
        k[:, h] = expand_keys(c, bf16_bits_to_f64(w_k_bits[h]))
        v[:, h] = expand_values(c, bf16_bits_to_f64(w_v_bits[h]))
    return k, v


def attention_on_expanded(q_bits_b: np.ndarray, k: np.ndarray, v: np.ndarray, cache_len: int, scale: float,
                          queries=None, heads=None):
    """Causal multi-head attention of one sequence's queries q_bits_b [Q, H, D] (bf16 bits) over
    given keys and values k, v [>= cache_len, H, D] (float64 values).  Query i sits at position
    cache_len - Q + i and sees positions j <= that.  Returns out [nq, nh, D], lse [nq, nh]."""
    Q, H, D = q_bits_b.shape
    qs = range(Q) if queries is None else list(queries)
    hs = range(H) if heads is None else list(heads)
    out = np.zeros((len(qs), len(hs), D))
    lse = np.zeros((len(qs), len(hs)))
    for iq, i in enumerate(qs):
        t = cache_len - Q + i
        for ih, h in enumerate(hs):
            o, l, _, _ = softmax_attention(bf16_bits_to_f64(q_bits_b[i, h]), k[: t + 1, h], v[: t + 1, h], scale)
            out[iq, ih] = o
            lse[iq, ih] = l
    return out, lse
