"""CPU oracle for the k-pooled sparse-attention indexer that produces the position lists
consumed by indexed latent attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the tests, the smoke check in __graft_entry__ and the cpu_baseline leg of bench.py
use it.  It shares no code with the HIP library.  Inputs are plain numpy arrays (bf16 values as
uint16 bit patterns, int32 lengths).

What the pages fix (colibri "GLM-5.3-Flash engine (c/glm53.c)", section "Architecture notes",
"DSA with k-pooling"; page "Module 08 -- Vision, MTP, and Hybrid Serving State", section 3 for
the pool-completion causality rule after rollback):
* indexer keys are grouped into pools of `pool` consecutive positions;
* a pool's key is a per-channel softmax mixture of its members' keys, not their mean;
* only a pool that is complete and causally visible can be selected;
* the incomplete tail pool is appended when asked for, which makes a row topk + pool - 1 wide;
* ties go to the lower index, so selection is deterministic.

Readings taken where the pages are silent:
* `topk` counts positions and is a multiple of `pool`: topk / pool pools are selected, each
  expanded to its `pool` positions (the only reading under which the row is topk + pool - 1
  wide); with fewer selectable pools, all of them are selected;
* the mixture weights are a softmax over the pool's positions of per-position, per-channel gate
  logits g, given as an input (the pages do not say where the logits come from);
* a pool's score for a query is the dot product of the indexer query with the pooled key;
* pool p (positions p*pool .. p*pool + pool - 1) is selectable by the query at position t when
  its last position is at most t; the tail is the positions floor((t+1)/pool)*pool .. t;
* the row lists the selected pools' positions in ascending order, then the tail; unused slots
  hold -1.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import bf16_bits_to_f64, query_position


def complete_pools(cache_len: int, pool: int) -> int:
    """Pools whose every member position lies inside a cache of cache_len positions (pool p holds
    positions p*pool .. p*pool + pool - 1)."""
    return int(cache_len) // int(pool)


def pooled_keys(k_bits: np.ndarray, g_bits: np.ndarray, pool: int, n_pools: int) -> np.ndarray:
    """Per-channel softmax mixture of each pool's keys (colibri "DSA with k-pooling").

    k_bits, g_bits: [L, d] bf16 bit patterns (keys and gate logits of one sequence).
    Returns [n_pools, d] float64: pooled[p, c] = sum_s w[s, c] k[s, c] over the pool's
    positions s, w[., c] = softmax over s of g[s, c] (max-subtracted)."""
    k = bf16_bits_to_f64(k_bits[: n_pools * pool]).reshape(n_pools, pool, -1)
    g = bf16_bits_to_f64(g_bits[: n_pools * pool]).reshape(n_pools, pool, -1)
    e = np.exp(g - g.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return (w * k).sum(axis=1)


def pool_scores(q_bits: np.ndarray, pooled: np.ndarray) -> np.ndarray:
    """Dot product of the indexer query [d] (bf16 bits) with every pooled key -> [n_pools]."""
    return pooled @ bf16_bits_to_f64(q_bits)


def select_positions(scores: np.ndarray, t: int, pool: int, topk: int, tail: bool) -> np.ndarray:
    """The position list of the query at position t: the topk // pool best complete, visible
    pools (ties to the lower pool index) in ascending order, expanded to positions, then the
    incomplete tail if asked for.  scores holds at least the selectable pools' scores."""
    if topk % pool:
        raise ValueError("topk must be a multiple of pool")
    n_sel = topk // pool
    selectable = (t + 1) // pool  # pools whose last position p*pool + pool - 1 <= t
    cand = np.arange(selectable)
    # order by descending score, then ascending pool index; keep the first n_sel
    order = sorted(cand.tolist(), key=lambda p: (-scores[p], p))
    chosen = sorted(order[:n_sel])
    rows = [np.arange(p * pool, p * pool + pool) for p in chosen]
    if tail:
        rows.append(np.arange(selectable * pool, t + 1))
    return np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)


def indexer_reference(q_bits: np.ndarray, k_bits: np.ndarray, g_bits: np.ndarray, cache_len: np.ndarray,
                      pool: int, topk: int, tail: bool = True):
    """Whole indexer for a batch.

    q_bits [B, Q, d], k_bits and g_bits [B, L_max, d] (bf16 bits), cache_len [B].  Query i of
    sequence b sits at position cache_len[b] - Q + i.  Returns (idx [B, Q, topk + pool - 1]
    int32 padded with -1, idx_len [B, Q] int32, scores: list per (b, i) of the float64 pool
    scores, for validity checks)."""
    B, Q, d = q_bits.shape
    width = topk + pool - 1
    idx = np.full((B, Q, width), -1, np.int32)
    idx_len = np.zeros((B, Q), np.int32)
    all_scores = []
    for b in range(B):
        L = int(cache_len[b])
        n_pools = complete_pools(L, pool)
        pk = pooled_keys(k_bits[b], g_bits[b], pool, n_pools)
        row_scores = []
        for i in range(Q):
            t = query_position(L, Q, i)
            s = pool_scores(q_bits[b, i], pk) if n_pools else np.zeros(0)
            sel = select_positions(s, t, pool, topk, tail) if t >= 0 else np.zeros(0, np.int32)
            idx[b, i, : sel.size] = sel
            idx_len[b, i] = sel.size
            row_scores.append(s)
        all_scores.append(row_scores)
    return idx, idx_len, all_scores
