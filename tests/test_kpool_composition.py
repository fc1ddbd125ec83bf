"""Pin of the k-pooled indexer oracle's composition (CPU only): the whole indexer_reference and
pool_scores against a brute force written with scalar loops from the rules the pages state.

colibri "GLM-5.3-Flash engine (c/glm53.c)", "Architecture notes", "DSA with k-pooling": keys are
pooled over groups of consecutive positions with a per-channel softmax mixture; a pool can be
chosen only once it is complete and causally visible; the incomplete tail is appended, which makes
a row topk + pool - 1 wide; ties go to the lower index.  "Module 08 -- Vision, MTP, and Hybrid
Serving State", section 3: after a rollback the selection is rebuilt under the same
pool-completion rule, so the lists depend only on the cache length and the query's position.
"Module 05 -- MLA: Compressing Per-Token History", section 4: a query sees positions up to its
own, and the Q tokens of a pass are the last Q positions of the cache.

The brute force shares nothing with the oracle but the bf16 widening: every exponential, sum,
dot product, comparison and list is a Python loop over scalars.  Each planted mistake (a query
position off by one either way, a pool count rounded up, scores from the plain mean of a pool's
keys) must make the comparison fail.
"""
import math

import numpy as np
import pytest

from mla_latent_cache_absorb_amd import workloads as wl
from oracle import kpool_indexer as kp
from oracle.mla_oracle import bf16_bits_to_f64


def bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def brute_indexer(q_bits, k_bits, g_bits, cache_len, pool, topk, tail):
    """Scalar-loop indexer: (idx [B][Q][topk + pool - 1] padded with -1, idx_len [B][Q],
    scores[b][i] = list of the scores of every complete pool of sequence b)."""
    B, Q, d = q_bits.shape
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    g = bf16_bits_to_f64(g_bits)
    width = topk + pool - 1
    idx = [[[-1] * width for _ in range(Q)] for _ in range(B)]
    idx_len = [[0] * Q for _ in range(B)]
    scores = []
    for b in range(B):
        L = int(cache_len[b])
        # a pool is complete when all of its members are cached positions
        pools = []
        p = 0
        while all(pos < L for pos in range(p * pool, p * pool + pool)):
            members = list(range(p * pool, p * pool + pool))
            key = []
            for c in range(d):
                top = max(g[b, s, c] for s in members)
                w = [math.exp(g[b, s, c] - top) for s in members]
                z = sum(w)
                key.append(sum(w[n] / z * k[b, s, c] for n, s in enumerate(members)))
            pools.append(key)
            p += 1
        # the pass's tokens are the last Q cached positions, in order
        new_positions = list(range(L))[L - Q:]
        row_scores = []
        for i in range(Q):
            t = new_positions[i]
            s = [sum(q[b, i, c] * key[c] for c in range(d)) for key in pools]
            row_scores.append(s)
            visible = [p for p in range(len(pools)) if p * pool + pool - 1 <= t]
            chosen = []
            for _ in range(topk // pool):
                best = None
                for p in visible:
                    if p in chosen:
                        continue
                    if best is None or s[p] > s[best]:
                        best = p          # strictly greater: the first (lowest) of equal scores stays
                if best is None:
                    break
                chosen.append(best)
            listed = []
            for p in sorted(chosen):
                listed += list(range(p * pool, p * pool + pool))
            if tail:
                # positions up to t whose pool is not yet selectable
                listed += [j for j in range(t + 1) if (j // pool) not in visible]
            for n, j in enumerate(listed):
                idx[b][i][n] = j
            idx_len[b][i] = len(listed)
        scores.append(row_scores)
    return np.array(idx, np.int32), np.array(idx_len, np.int32), scores


def make_inputs(seed, B, Q, L_max, d, tie_pools=False):
    rng = np.random.default_rng(seed)
    q = bits(rng.standard_normal((B, Q, d)))
    k = bits(rng.standard_normal((B, L_max, d)))
    g = bits(rng.standard_normal((B, L_max, d)) * 2.0)
    if tie_pools:
        # every pool of sequence 0 holds the same keys and gates: all its pool scores are equal
        k[0] = k[0, :1]
        g[0] = g[0, :1]
    return q, k, g


CASES = [
    # seed, lengths (ragged; pool sizes leave tails), Q, pool, topk, tail
    (11, [23, 18, 30], 3, 4, 8, True),
    (12, [23, 18, 30], 4, 4, 8, False),
    (13, [17, 9, 26], 3, 3, 6, True),
    (14, [40, 12, 33], 5, 4, 64, True),   # topk above the selectable pools: all of them are chosen
    (15, [21, 22, 24], 3, 2, 4, True),
]


def compare(got, want):
    idx, n, sc = got
    widx, wn, wsc = want
    np.testing.assert_array_equal(n, wn)
    np.testing.assert_array_equal(idx, widx)
    for b in range(len(wsc)):
        for i in range(len(wsc[b])):
            assert len(sc[b][i]) == len(wsc[b][i]), (b, i, len(sc[b][i]), len(wsc[b][i]))
            np.testing.assert_allclose(sc[b][i], wsc[b][i], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed,lens,Q,pool,topk,tail", CASES)
def test_indexer_matches_brute_force(seed, lens, Q, pool, topk, tail):
    B, d = len(lens), 8
    q, k, g = make_inputs(seed, B, Q, max(lens) + 5, d)
    lens = np.array(lens, np.int32)
    got = kp.indexer_reference(q, k, g, lens, pool, topk, tail)
    compare(got, brute_indexer(q, k, g, lens, pool, topk, tail))
    # pool_scores on its own: one query's scores of every complete pool of sequence 0
    n_pools = int(lens[0]) // pool
    s = kp.pool_scores(q[0, 0], kp.pooled_keys(k[0], g[0], pool, n_pools))
    np.testing.assert_allclose(s, brute_indexer(q, k, g, lens, pool, topk, tail)[2][0][0], rtol=1e-12, atol=1e-12)


def test_equal_scores_choose_the_lowest_pools():
    q, k, g = make_inputs(21, 2, 3, 40, 8, tie_pools=True)
    lens = np.array([37, 29], np.int32)
    got = kp.indexer_reference(q, k, g, lens, 4, 12, True)
    want = brute_indexer(q, k, g, lens, 4, 12, True)
    compare(got, want)
    # with every pool equal, sequence 0's queries list pools 0, 1, 2 and then their tail
    assert list(got[0][0, 0, :12]) == list(range(12))


def test_query_positions_match_single_token_steps():
    # query i of a Q-token pass at cache length L lists what a one-token step at length L - Q + i + 1
    # lists: its own position is the last cached one (time consistency after a rollback)
    q, k, g = make_inputs(31, 2, 4, 48, 8)
    lens = np.array([43, 26], np.int32)
    idx, n, _ = kp.indexer_reference(q, k, g, lens, 4, 8, True)
    for b in range(2):
        for i in range(4):
            step_len = np.array([lens[b] - 4 + i + 1], np.int32)
            i1, n1, _ = kp.indexer_reference(q[b:b + 1, i:i + 1], k[b:b + 1], g[b:b + 1], step_len, 4, 8, True)
            assert n1[0, 0] == n[b, i]
            np.testing.assert_array_equal(i1[0, 0], idx[b, i])
            # while its pool is incomplete the query's own position ends its list (the tail)
            t = lens[b] - 4 + i
            if (t + 1) % 4:
                assert idx[b, i, n[b, i] - 1] == t
            assert idx[b, i, :n[b, i]].max() < lens[b]


# --------------------------------------------------------------------------- planted mistakes
def _assert_some_case_fails():
    failed = 0
    for case in CASES:
        try:
            test_indexer_matches_brute_force(*case)
        except (AssertionError, IndexError, ValueError):  # a wrong result, or the oracle refusing its own output
            failed += 1
    assert failed > 0, "the planted mistake passed every case"


def test_planted_late_query_position_fails(monkeypatch):
    monkeypatch.setattr(kp, "query_position", lambda L, Q, i: int(L) - int(Q) + int(i) + 1)
    _assert_some_case_fails()


def test_planted_early_query_position_fails(monkeypatch):
    monkeypatch.setattr(kp, "query_position", lambda L, Q, i: int(L) - int(Q) + int(i) - 1)
    _assert_some_case_fails()


def test_planted_rounded_up_pool_count_fails(monkeypatch):
    monkeypatch.setattr(kp, "complete_pools", lambda L, pool: -(-int(L) // int(pool)))
    _assert_some_case_fails()


def test_planted_mean_pooled_scores_fail(monkeypatch):
    def mean_pooled(k_bits, g_bits, pool, n_pools):
        return bf16_bits_to_f64(k_bits[: n_pools * pool]).reshape(n_pools, pool, -1).mean(axis=1)
    monkeypatch.setattr(kp, "pooled_keys", mean_pooled)
    _assert_some_case_fails()
