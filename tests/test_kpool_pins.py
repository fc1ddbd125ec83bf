"""Pins of the k-pooled indexer oracle to facts the pages and mathematics fix (CPU only).

colibri "GLM-5.3-Flash engine (c/glm53.c)", "Architecture notes", "DSA with k-pooling": pooled
keys are per-channel softmax mixtures, only complete and causally visible pools are selectable,
the incomplete tail is appended (rows topk + pool - 1 wide), ties go to the lower index.
"""
import json
import os

import numpy as np
import pytest

from mla_latent_cache_absorb_amd import workloads as wl
from oracle import kpool_indexer as kp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kpool_row_width.json")


def bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def rand_bits(rng, shape, scale=1.0):
    return bits(rng.standard_normal(shape).astype(np.float32) * scale)


def test_equal_gates_give_the_mean():
    # softmax of equal logits is uniform: the mixture reduces to the plain mean
    rng = np.random.default_rng(1)
    k = rand_bits(rng, (16, 8))
    g = bits(np.full((16, 8), 0.375))
    pooled = kp.pooled_keys(k, g, 4, 4)
    kf = kp.bf16_bits_to_f64(k).reshape(4, 4, 8)
    np.testing.assert_allclose(pooled, kf.mean(axis=1), rtol=1e-12, atol=1e-12)


def test_dominant_gate_selects_per_channel():
    # a gate logit far above the others in one channel picks that position's key for that
    # channel only: channels of one pool may take different members (not the pool mean)
    rng = np.random.default_rng(2)
    k = rand_bits(rng, (4, 3))
    g = np.zeros((4, 3), np.float32)
    g[1, 0] = 60.0
    g[3, 1] = 60.0
    g[0, 2] = 60.0
    pooled = kp.pooled_keys(k, bits(g), 4, 1)[0]
    kf = kp.bf16_bits_to_f64(k)
    np.testing.assert_allclose(pooled, [kf[1, 0], kf[3, 1], kf[0, 2]], rtol=1e-20, atol=1e-20)
    assert not np.allclose(pooled, kf.mean(axis=0))


def _select_by_repeated_argmax(scores, t, pool, topk, tail):
    # independent selection: take the best remaining pool n times (first occurrence wins ties)
    s = list(scores[: (t + 1) // pool])
    taken = []
    for _ in range(min(topk // pool, len(s))):
        best = None
        for p, v in enumerate(s):
            if p in taken:
                continue
            if best is None or v > s[best]:
                best = p
        taken.append(best)
    pos = [q for p in sorted(taken) for q in range(p * pool, p * pool + pool)]
    if tail:
        pos += list(range((t + 1) // pool * pool, t + 1))
    return np.array(pos, np.int32)


@pytest.mark.parametrize("pool,topk,L", [(4, 16, 64), (2, 6, 17), (8, 16, 41), (4, 8, 5), (4, 400, 64)])
def test_selection_matches_repeated_argmax(pool, topk, L):
    rng = np.random.default_rng(pool * 100 + topk)
    for t in range(L):
        scores = np.round(rng.standard_normal(L // pool) * 4) / 4  # coarse values: many ties
        for tail in (False, True):
            got = kp.select_positions(scores, t, pool, topk, tail)
            want = _select_by_repeated_argmax(scores, t, pool, topk, tail)
            np.testing.assert_array_equal(got, want)


def test_causality_and_row_width():
    spec = json.load(open(GOLDEN))
    rng = np.random.default_rng(3)
    for row in spec["rows"]:
        topk, pool, width = row["topk"], row["pool"], row["width"]
        scores = rng.standard_normal(4096)
        for t in (topk * 3 + pool - 1, topk * 3 + pool - 2, topk * 3 + pool):
            sel = kp.select_positions(scores, t, pool, topk, True)
            assert sel.size <= width
            assert sel.max() <= t and np.all(np.diff(sel) > 0)
            # every selected position outside the tail belongs to a complete pool
            n_tail = (t + 1) % pool
            body = sel[: sel.size - n_tail]
            assert body.size == topk and np.all(body.reshape(-1, pool) // pool == (body.reshape(-1, pool)[:, :1] // pool))
            assert np.all(body.reshape(-1, pool)[:, -1] <= t)
        # a pool whose last position equals t is selectable; one position short is not
        t = 2 * pool - 1
        s = np.zeros(2)
        s[1] = 5.0
        assert (2 * pool - 1) in kp.select_positions(s, t, pool, pool, False)
        assert kp.select_positions(s, t - 1, pool, pool, False).max() == pool - 1
    assert max(r["width"] for r in spec["rows"] if r["pool"] == 4) == 2051


def test_ties_go_to_the_lower_pool():
    scores = np.zeros(10)
    sel = kp.select_positions(scores, 39, 4, 12, False)
    np.testing.assert_array_equal(sel, np.arange(12))


def test_short_history_selects_every_complete_pool():
    sel = kp.select_positions(np.arange(3.0), 13, 4, 64, True)
    np.testing.assert_array_equal(sel, np.arange(14))


def test_rows_past_cache_len_are_never_read():
    rng = np.random.default_rng(4)
    B, Q, L, d = 2, 3, 50, 8
    q = rand_bits(rng, (B, Q, d))
    k = rand_bits(rng, (B, L + 20, d))
    g = rand_bits(rng, (B, L + 20, d))
    lens = np.array([L, 37], np.int32)
    idx, n, _ = kp.indexer_reference(q, k, g, lens, 4, 8)
    k2, g2 = k.copy(), g.copy()
    for b in range(B):
        k2[b, lens[b]:] = wl.BF16_NAN
        g2[b, lens[b]:] = wl.BF16_NAN
    idx2, n2, _ = kp.indexer_reference(q, k2, g2, lens, 4, 8)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(n, n2)


PLANTED = {
    "mean_pooling": lambda k, g, pool, n: kp.bf16_bits_to_f64(k[: n * pool]).reshape(n, pool, -1).mean(axis=1),
}


def test_planted_mean_pooling_fails_the_gate_pin(monkeypatch):
    monkeypatch.setattr(kp, "pooled_keys", PLANTED["mean_pooling"])
    with pytest.raises(AssertionError):
        test_dominant_gate_selects_per_channel()


def test_planted_off_by_one_causality_fails(monkeypatch):
    orig = kp.select_positions

    def late(scores, t, pool, topk, tail):
        return orig(scores, t + 1, pool, topk, tail)[:-1] if tail else orig(scores, t + 1, pool, topk, tail)
    monkeypatch.setattr(kp, "select_positions", late)
    with pytest.raises(AssertionError):
        test_selection_matches_repeated_argmax(2, 6, 17)


def test_planted_ties_to_higher_index_fail(monkeypatch):
    def high(scores, t, pool, topk, tail):
        sel = (t + 1) // pool
        order = sorted(range(sel), key=lambda p: (-scores[p], -p))[: topk // pool]
        pos = [q for p in sorted(order) for q in range(p * pool, p * pool + pool)]
        if tail:
            pos += list(range(sel * pool, t + 1))
        return np.array(pos, np.int32)
    monkeypatch.setattr(kp, "select_positions", high)
    with pytest.raises(AssertionError):
        test_ties_go_to_the_lower_pool()
