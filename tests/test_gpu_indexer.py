"""GPU parity of the k-pooled indexer (called through the C ABI) against the fp64 CPU oracle.

Pooled keys and scores are floating point: held to a bound from fp32 rounding.  The selection
is integer work decided on the kernel's fp32 scores, so it is checked bit for bit against the
oracle's selection rule applied to those same scores (both sides decide in fp32); on inputs
whose arithmetic is exact in fp32 the whole indexer is checked bit for bit against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import kpool_indexer as kp
from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import DEV, assert_parity, bf16, i32

pytestmark = pytest.mark.gpu

F = oracle.bf16_bits_to_f64


def bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def run_indexer(q, k, g, lens, pool, topk, tail=True, max_cache_len=None):
    L = int(max_cache_len or k.shape[1])
    cl = i32(lens)
    pooled = binding.mla_kpool_keys(bf16(k), bf16(g), cl, L, pool)
    scores = binding.mla_indexer_scores(bf16(q), pooled, cl, L, pool)
    idx, n = binding.mla_indexer_select(scores, cl, L, pool, topk, tail)
    torch.cuda.synchronize()
    return pooled.cpu().numpy(), scores.cpu().numpy(), idx.cpu().numpy(), n.cpu().numpy()


def oracle_select_on(scores, lens, Q, pool, topk, tail, width):
    B = scores.shape[0]
    idx = np.full((B, Q, width), -1, np.int32)
    n = np.zeros((B, Q), np.int32)
    for b in range(B):
        for i in range(Q):
            t = int(lens[b]) - Q + i
            sel = kp.select_positions(scores[b, i].astype(np.float64), t, pool, topk, tail)
            idx[b, i, :sel.size] = sel
            n[b, i] = sel.size
    return idx, n


@pytest.mark.parametrize("pool,topk,tail", [(4, 16, True), (4, 16, False), (2, 6, True), (8, 64, True), (16, 64, True)])
def test_exact_inputs_bit_exact(pool, topk, tail):
    # small integers and equal gates: pooling is an exact mean, scores exact integers with
    # many ties, so the whole indexer must match the oracle bit for bit
    rng = np.random.default_rng(pool * 10 + topk)
    B, Q, Lm, d = 3, 4, 203, 128
    lens = np.array([203, 150, 37], np.int32)
    q = bits(rng.integers(-2, 3, (B, Q, d)))
    k = bits(rng.integers(-4, 5, (B, Lm, d)) * pool)  # multiples of the pool: the mean stays an integer
    g = bits(np.full((B, Lm, d), 1.5))
    pooled, scores, idx, n = run_indexer(q, k, g, lens, pool, topk, tail)
    ridx, rn, rs = kp.indexer_reference(q, k, g, lens, pool, topk, tail)
    np.testing.assert_array_equal(n, rn)
    np.testing.assert_array_equal(idx, ridx[:, :, : idx.shape[2]])
    for b in range(B):
        npb = lens[b] // pool
        np.testing.assert_array_equal(scores[b, :, :npb], np.array(rs[b]))


def test_random_inputs_scores_and_selection():
    rng = np.random.default_rng(7)
    B, Q, Lm, d, pool, topk = 2, 6, 1500, 128, 4, 64
    lens = np.array([1500, 999], np.int32)
    q, k, g = rand = (bits(rng.standard_normal((B, Q, d))), bits(rng.standard_normal((B, Lm, d))),
                      bits(rng.standard_normal((B, Lm, d)) * 2))
    for b in range(B):
        k[b, lens[b]:] = wl.BF16_NAN
        g[b, lens[b]:] = wl.BF16_NAN
    pooled, scores, idx, n = run_indexer(q, k, g, lens, pool, topk)
    for b in range(B):
        npb = lens[b] // pool
        ref = kp.pooled_keys(k[b], g[b], pool, npb)
        assert np.abs(pooled[b, :npb] - ref).max() <= 1e-5 * np.abs(ref).max() + 1e-6
        rs = np.stack([kp.pool_scores(q[b, i], ref) for i in range(Q)])
        bound = 1e-5 * (np.abs(F(q[b])) @ np.abs(ref).T).max() + 1e-5
        assert np.abs(scores[b, :, :npb] - rs).max() <= bound
    ridx, rn = oracle_select_on(scores, lens, Q, pool, topk, True, topk + pool - 1)
    np.testing.assert_array_equal(n, rn)
    np.testing.assert_array_equal(idx, ridx)


def test_indexer_feeds_indexed_attention():
    # indexer -> indexed latent attention, against the oracle's attention over the same lists
    spec = wl.make_spec(2, 4, 900, min_cache_len=500, workload_id=640)
    w = wl.make_workload(spec)
    ix = wl.make_indexer_inputs(spec, w.cache_len, d=128, pool=4, topk=128)
    cl = i32(w.cache_len)
    idx, n = binding.mla_indexer(bf16(ix.q), bf16(ix.k), bf16(ix.g), cl, 900, 4, 128)
    qa = wl.latent_query_bits(spec)
    o, lse = binding.mla_latent_attn_indexed(bf16(qa), bf16(w.cache), cl, idx, n, 900, w.scale, 0)
    torch.cuda.synchronize()
    idx_h, n_h = idx.cpu().numpy(), n.cpu().numpy()
    ref, lse_ref = oracle.latent_attention(F(qa), w.cache, w.cache_len, w.scale, idx=idx_h, idx_len=n_h)
    assert_parity(o.cpu().numpy(), ref, "indexer -> indexed attention")
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=1e-3)


def test_rollback_and_incremental_pools():
    # truncating cache_len equals a run on a cache that never held the removed rows, and
    # building only the pools completed by new positions equals a full rebuild
    rng = np.random.default_rng(9)
    B, Q, Lm, d, pool, topk = 2, 2, 600, 128, 4, 32
    q = bits(rng.standard_normal((B, Q, d)))
    k = bits(rng.standard_normal((B, Lm, d)))
    g = bits(rng.standard_normal((B, Lm, d)))
    full = np.array([600, 437], np.int32)
    short = np.array([553, 420], np.int32)
    _, _, idx_a, n_a = run_indexer(q, k, g, short, pool, topk)
    k2, g2 = k.copy(), g.copy()
    for b in range(B):
        k2[b, short[b]:] = wl.BF16_NAN
        g2[b, short[b]:] = wl.BF16_NAN
    _, _, idx_b, n_b = run_indexer(q, k2, g2, short, pool, topk)
    np.testing.assert_array_equal(idx_a, idx_b)
    np.testing.assert_array_equal(n_a, n_b)
    # incremental: pools of the short caches first, then only the pools the rest completes
    kt, gt = bf16(k), bf16(g)
    pooled = binding.mla_kpool_keys(kt, gt, i32(short), Lm, pool, max_pools=Lm // pool)
    binding.mla_kpool_keys(kt, gt, i32(full), Lm, pool, pooled=pooled, pool_begin=i32(short // pool))
    whole = binding.mla_kpool_keys(kt, gt, i32(full), Lm, pool)
    torch.cuda.synchronize()
    for b in range(B):
        npb = full[b] // pool
        np.testing.assert_array_equal(pooled[b, :npb].cpu().numpy(), whole[b, :npb].cpu().numpy())


def test_full_size_sampled():
    # the indexed verification shape: 32 sequences of 4096..65536 positions, 4 queries each,
    # pool 4, 2048 positions selected; selection exact against the oracle rule on the kernel's
    # scores for every query, scores against fp64 on sampled sequences
    spec = wl.WORKLOADS["indexed_verify_b32_q4_ragged"]
    lens = wl.cache_lengths(spec)
    ix = wl.make_indexer_inputs(spec, lens)
    pooled, scores, idx, n = run_indexer(ix.q, ix.k, ix.g, lens, ix.pool, ix.topk)
    ridx, rn = oracle_select_on(scores, lens, spec.q_len, ix.pool, ix.topk, True, ix.topk + ix.pool - 1)
    np.testing.assert_array_equal(n, rn)
    np.testing.assert_array_equal(idx, ridx)
    for b in (0, 17):
        npb = lens[b] // ix.pool
        ref = kp.pooled_keys(ix.k[b], ix.g[b], ix.pool, npb)
        assert np.abs(pooled[b, :npb] - ref).max() <= 1e-5 * np.abs(ref).max() + 1e-6
        rs = np.stack([kp.pool_scores(ix.q[b, i], ref) for i in range(spec.q_len)])
        bound = 1e-5 * (np.abs(F(ix.q[b])) @ np.abs(ref).T).max() + 1e-5
        assert np.abs(scores[b, :, :npb] - rs).max() <= bound


@pytest.mark.parametrize("kind", ["all_equal", "three_levels", "ties_at_threshold"])
def test_selection_ties_across_the_whole_row(kind):
    # up to 16384 selectable pools: the tie group at the threshold spans many threads' pool
    # ranges, and the lowest-index-first rule must still hold exactly
    rng = np.random.default_rng(21)
    B, Q, pool, topk = 2, 2, 4, 2048
    L = np.array([65536, 40001], np.int32)
    n_pools = 65536 // pool
    if kind == "all_equal":
        s = np.zeros((B, Q, n_pools), np.float32)
    elif kind == "three_levels":
        s = rng.integers(0, 3, (B, Q, n_pools)).astype(np.float32) - 1.0
    else:
        s = rng.standard_normal((B, Q, n_pools)).astype(np.float32)
        s[s > 2.2] = 2.2  # a large tie group right at the 512th-largest value
    idx, n = binding.mla_indexer_select(torch.from_numpy(s).to(DEV), i32(L), 65536, pool, topk, True)
    torch.cuda.synchronize()
    ridx, rn = oracle_select_on(s, L, Q, pool, topk, True, topk + pool - 1)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)


@pytest.mark.parametrize("d,Q", [(64, 3), (64, 8), (128, 6), (256, 2), (256, 5)])
def test_exact_inputs_every_width(d, Q):
    # every key width and query count the scores kernel specialises on (queries held in
    # registers or read from LDS), bit for bit against the oracle on exact inputs
    rng = np.random.default_rng(d * 10 + Q)
    B, Lm, pool, topk = 2, 150, 4, 16
    lens = np.array([150, 61], np.int32)
    q = bits(rng.integers(-2, 3, (B, Q, d)))
    k = bits(rng.integers(-4, 5, (B, Lm, d)) * pool)
    g = bits(np.full((B, Lm, d), -0.75))
    pooled, scores, idx, n = run_indexer(q, k, g, lens, pool, topk, True)
    ridx, rn, rs = kp.indexer_reference(q, k, g, lens, pool, topk, True)
    np.testing.assert_array_equal(n, rn)
    np.testing.assert_array_equal(idx, ridx[:, :, : idx.shape[2]])
    for b in range(B):
        npb = lens[b] // pool
        np.testing.assert_array_equal(scores[b, :, :npb], np.array(rs[b]))
