"""CPU oracle for absorbed Multi-head Latent Attention over a latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check in __graft_entry__ and
the cpu_baseline leg of bench.py use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants); its only input is
plain numpy arrays (bf16 values as uint16 bit patterns, int32 lengths and
positions), as produced by the seeded workload generators.

It is written in plain numpy, in float64, following the pages:

* "Module 05 -- MLA: Compressing Per-Token History" (jared-hpc.com,
  GLM-5.3-Flash Architecture Mastery, Lecture-05):
  - section 1 (The latent representation): each token j is cached as ONE
    latent c_j of width 512; per-head keys and values are rebuilt from it by
    per-head up-projections, k_{j,h} = U_h^K c_j and v_{j,h} = U_h^V c_j
    (the formulas after the colons are missing from the extracted text; the
    relations are restated intact in the substitution steps of section 3 and in
    colibri's "MLA is absorbed" section);
  - section 2 (The memory advantage, derived): 65,536 bytes per token per
    layer expanded against 1,024 as a latent, a 64x ratio;
  - section 3 (The algebra that avoids re-expanding history): the absorbed
    query (U_h^K)^T q_h, scores as dot products with the cached latent, the
    value sum accumulated in latent space and expanded once by U_h^V; and the
    rule that the absorbed form must reproduce the SAME score values
    (same softmax scale), not proportional ones;
  - section 4 (NoPE does not mean order-blind): no rotary terms; causal
    masking lets a query see only positions j <= t;
  - section 5 (Prefill and decode may want different algebra): the NAIVE form
    (expand every historical k, v, then ordinary multi-head attention) and the
    ABSORBED form.
* colibri "GLM-5.3-Flash engine (c/glm53.c)", section "MLA is absorbed": the
  two identities score_j = q.(W_k c_j) = (W_k^T q).c_j and
  out = sum_j a_j (W_v c_j) = W_v (sum_j a_j c_j); the absorbed form is exact,
  only the order of the products changes.
* "Module 08 -- Vision, MTP, and Hybrid Serving State", section 2 (the full
  model verifies the drafted tokens in one forward pass) and section 3 (the MLA
  latent cache is truncatable by position).

Reference computation (`mla_reference`) is the NAIVE/expanded form: it expands
k and v for every visible position and runs textbook max-subtracted softmax
attention.  The absorbed-form stages (`absorbed_query`, `latent_attention`,
`up_project`) are given too, as plain definitions, so each library stage can be
checked on its own.

Readings taken where the pages are silent:
* query i (0-based) of a pass of Q new positions sits at position
  cache_len - Q + i and its own latent is already in the cache; it sees every
  position j <= that position (inclusive, "only j <= t");
* weights are stored per head as [H][D][R] (row h is U_h as a D x R matrix);
* the softmax scale multiplies q.k (1/16 for the 256-wide heads);
* lse is the natural log of sum_j exp(scale * q.k_j);
* the indexed variant attends exactly to the given sorted, unique, causal
  positions.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64: a bf16 value is the top 16 bits
    of the float32 with the same sign, exponent and leading mantissa bits."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# visible sets (integer work; Module 05 section 4: only j <= t)
# --------------------------------------------------------------------------
def query_position(cache_len: int, q_len: int, i: int) -> int:
    """Position of query i among the Q new positions whose latents end the cache."""
    return int(cache_len) - int(q_len) + int(i)


def dense_visible_positions(cache_len: int, q_len: int, i: int) -> np.ndarray:
    """Causal visible set of query i: every cached position j <= its own position."""
    t = query_position(cache_len, q_len, i)
    if t < 0:
        raise ValueError("query position before the start of the cache")
    return np.arange(0, t + 1, dtype=np.int64)


def indexed_visible_positions(idx_row: np.ndarray, n: int, cache_len: int, q_len: int, i: int) -> np.ndarray:
    """Visible set of query i in the indexed variant: exactly idx_row[:n], which must be sorted,
    unique and causal (every position <= the query's own position)."""
    t = query_position(cache_len, q_len, i)
    sel = np.asarray(idx_row[: int(n)], dtype=np.int64)
    if sel.size == 0:
        raise ValueError("empty visible set")
    if np.any(np.diff(sel) <= 0):
        raise ValueError("index set must be sorted and unique")
    if sel[0] < 0 or sel[-1] > t:
        raise ValueError("index set must be causal and inside the cache")
    return sel


def visible_sets(cache_len_b: int, q_len: int, idx_b=None, idx_len_b=None, queries=None):
    """{query i: sorted visible positions} for one sequence."""
    queries = range(q_len) if queries is None else queries
    out = {}
    for i in queries:
        if idx_b is None:
            out[i] = dense_visible_positions(cache_len_b, q_len, i)
        else:
            out[i] = indexed_visible_positions(idx_b[i], idx_len_b[i], cache_len_b, q_len, i)
    return out


# --------------------------------------------------------------------------
# the naive (expanded) form -- the reference result
# --------------------------------------------------------------------------
def expand_keys(c: np.ndarray, w_k_h: np.ndarray) -> np.ndarray:
    """k_{j,h} = U_h^K c_j for every row c_j of c [T, R]; U_h^K is w_k_h [D, R].  Returns [T, D]."""
    return c @ w_k_h.T


def expand_values(c: np.ndarray, w_v_h: np.ndarray) -> np.ndarray:
    """v_{j,h} = U_h^V c_j for every row c_j of c [T, R]; U_h^V is w_v_h [D, R].  Returns [T, D]."""
    return c @ w_v_h.T


def softmax_attention(q_h: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Textbook attention of one query against T keys/values:
    s_j = scale * q.k_j; a = exp(s - max s) / sum exp(s - max s); out = sum_j a_j v_j.
    Returns (out [D], lse, s [T], a [T]) with lse = max s + ln sum exp(s - max s).
    q_h may also be [n, D], n queries against the same keys and values: each is one column of
    s and a ([T, n]), and out is [n, D], lse [n]."""
    s = scale * (k @ np.asarray(q_h).T)
    m = s.max(axis=0)
    e = np.exp(s - m)
    z = e.sum(axis=0)
    a = e / z
    return a.T @ v, m + np.log(z), s, a


def _select(seq: Optional[Iterable[int]], n: int) -> list:
    return list(range(n)) if seq is None else [int(x) for x in seq]


def mla_reference(q_bits, cache_bits, w_k_bits, w_v_bits, cache_len, scale, *, idx=None, idx_len=None,
                  batches: Optional[Sequence[int]] = None, queries: Optional[Sequence[int]] = None,
                  heads: Optional[Sequence[int]] = None):
    """Reference output of MLA attention in the naive form (Module 05 section 5), fp64.

    q_bits [B, Q, H, D], cache_bits [B, L_max, R], w_*_bits [H, D, R] (bf16 bits); cache_len [B];
    idx [B, Q, K_max] / idx_len [B, Q] select the indexed variant.  Optional subsets of batches,
    queries and heads restrict the work (sampled parity at full sizes).
    Returns out [nb, nq, nh, D] and lse [nb, nq, nh] (float64), in the order of the subsets.
    """
    B, Q, H, D = q_bits.shape
    bs, qs, hs = _select(batches, B), _select(queries, Q), _select(heads, H)
    out = np.zeros((len(bs), len(qs), len(hs), D))
    lse = np.zeros((len(bs), len(qs), len(hs)))
    for ib, b in enumerate(bs):
        vis = visible_sets(int(cache_len[b]), Q,
                           None if idx is None else idx[b], None if idx_len is None else idx_len[b], qs)
        union = np.unique(np.concatenate([vis[i] for i in qs]))
        c = bf16_bits_to_f64(cache_bits[b, union])            # [U, R]
        for ih, h in enumerate(hs):
            k = expand_keys(c, bf16_bits_to_f64(w_k_bits[h]))    # [U, D]
            v = expand_values(c, bf16_bits_to_f64(w_v_bits[h]))  # [U, D]
            for iq, i in enumerate(qs):
                rows = np.searchsorted(union, vis[i])
                o, l, _, _ = softmax_attention(bf16_bits_to_f64(q_bits[b, i, h]), k[rows], v[rows], scale)
                out[ib, iq, ih] = o
                lse[ib, iq, ih] = l
    return out, lse


def expanded_scores(q_bits, cache_bits, w_k_bits, scale, b, i, h, positions) -> np.ndarray:
    """Scores of the naive form for one (sequence, query, head): scale * q_h . (U_h^K c_j)."""
    c = bf16_bits_to_f64(cache_bits[b, np.asarray(positions)])
    k = expand_keys(c, bf16_bits_to_f64(w_k_bits[h]))
    return scale * (k @ bf16_bits_to_f64(q_bits[b, i, h]))


# --------------------------------------------------------------------------
# the absorbed-form stages, each its plain definition (Module 05 section 3;
# colibri "MLA is absorbed")
# --------------------------------------------------------------------------
def absorbed_query(q_bits, w_k_bits) -> np.ndarray:
    """q~_h = (U_h^K)^T q_h for every query row and head.  q_bits [..., H, D] -> [..., H, R] fp64."""
    q = bf16_bits_to_f64(q_bits)
    w = bf16_bits_to_f64(w_k_bits)                          # [H, D, R]
    out = np.empty(q.shape[:-1] + (w.shape[2],))
    for h in range(w.shape[0]):
        out[..., h, :] = q[..., h, :] @ w[h]                # (U^T q)_r = sum_d U[d, r] q[d]
    return out


def latent_attention(q_abs, cache_bits, cache_len, scale, *, idx=None, idx_len=None,
                     batches=None, queries=None, heads=None):
    """Attention read directly from the cached latents, given absorbed queries q_abs [B, Q, H, R]
    (float64 values, e.g. widened bf16 bits): s_j = scale * q~_h . c_j; a = softmax(s) over the
    visible set; o_lat = sum_j a_j c_j (accumulated in latent space).
    Returns o_lat [nb, nq, nh, R] and lse [nb, nq, nh]."""
    B, Q, H, R = q_abs.shape
    bs, qs, hs = _select(batches, B), _select(queries, Q), _select(heads, H)
    o_lat = np.zeros((len(bs), len(qs), len(hs), R))
    lse = np.zeros((len(bs), len(qs), len(hs)))
    for ib, b in enumerate(bs):
        vis = visible_sets(int(cache_len[b]), Q,
                           None if idx is None else idx[b], None if idx_len is None else idx_len[b], qs)
        for iq, i in enumerate(qs):
            c = bf16_bits_to_f64(cache_bits[b, vis[i]])      # [T, R]
            # every requested head of the query against the same cached latents (K = V = c)
            o, l, _, _ = softmax_attention(np.asarray(q_abs[b, i, hs], np.float64), c, c, scale)
            o_lat[ib, iq] = o
            lse[ib, iq] = l
    return o_lat, lse


def up_project(o_lat, w_v_bits) -> np.ndarray:
    """out_h = U_h^V o_lat,h: the single expansion of the accumulated latent.
    o_lat [..., H, R] (float64) -> [..., H, D]."""
    w = bf16_bits_to_f64(w_v_bits)                          # [H, D, R]
    o = np.asarray(o_lat, np.float64)
    out = np.empty(o.shape[:-1] + (w.shape[1],))
    for h in range(w.shape[0]):
        out[..., h, :] = o[..., h, :] @ w[h].T
    return out


# --------------------------------------------------------------------------
# cache arithmetic (Module 05 section 2)
# --------------------------------------------------------------------------
def cache_bytes_per_token(heads: int, head_dim: int, latent: int, bytes_per_value: int = 2):
    """(expanded, latent) bytes per token per layer: the expanded cache stores a key and a value of
    head_dim per head; the latent cache stores one latent vector."""
    expanded = heads * head_dim * 2 * bytes_per_value
    lat = latent * bytes_per_value
    return expanded, lat
