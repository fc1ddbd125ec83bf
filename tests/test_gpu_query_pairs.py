"""GPU parity of the query-pair split kernel: dense calls with an even number of queries per
sequence run adjacent queries (i0 = i1 + 1) in one workgroup over one run of tiles.

The two queries differ only in their last visible position (page "Module 05 -- MLA: Compressing
Per-Token History", section 4: query i sees positions up to cache_len - Q + i), so the later
query's extra position must be masked out of the earlier one's scores, and a split holding only
that position must give the earlier query an empty partial.  The indexed call runs the
single-query kernel with the same splits, tiles and arithmetic order; listing every causal
position must reproduce the dense call bit for bit.  Lengths are chosen so that the later query's
last position opens a split or a tile of its own, and the results are checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import assert_parity, bf16, i32

pytestmark = pytest.mark.gpu

F = oracle.bf16_bits_to_f64

# max_cache_len 400 is 13 tiles; three splits hold 5, 5 and 3 tiles (160 positions each).
# Lengths 161 and 321 leave the later query of the last pair alone in the last split; 193 puts its
# last position alone in a tile; 400 fills the cache.
LENS = [161, 321, 193, 400]


def full_causal_lists(lens, Q, K):
    idx = np.full((len(lens), Q, K), -1, np.int32)
    idx_len = np.zeros((len(lens), Q), np.int32)
    for b, L in enumerate(lens):
        for i in range(Q):
            n = max(L - Q + i + 1, 0)
            idx[b, i, :n] = np.arange(n)
            idx_len[b, i] = n
    return idx, idx_len


@pytest.mark.parametrize("Q", [2, 4, 6, 8])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_pairs_equal_single_query_kernel_and_oracle(Q, splits):
    Lmax = 400
    spec = wl.make_spec(len(LENS), Q, Lmax, workload_id=1300 + Q)
    w = wl.make_workload(spec)
    lens = np.array(LENS, np.int32)
    w.cache_len[:] = lens
    for b, L in enumerate(lens):
        w.cache[b, L:] = wl.BF16_NAN
    qa_bits = wl.latent_query_bits(spec)
    qa, c, cl = bf16(qa_bits), bf16(w.cache), i32(lens)
    idx, idx_len = full_causal_lists(lens, Q, Lmax)
    # the automatic choice counts workgroups, which pairs make fewer for the dense call: both calls
    # are given the dense call's split count, so that they share the schedule
    s = binding.mla_latent_attn_num_splits(len(LENS), Q, 64, Lmax, splits)
    print(f"pairs Q={Q} splits={splits} -> {s}", flush=True)
    dense, ld = binding.mla_latent_attn(qa, c, cl, Lmax, w.scale, s)
    ind, li = binding.mla_latent_attn_indexed(qa, c, cl, i32(idx), i32(idx_len), Lmax, w.scale, s)
    torch.cuda.synchronize()
    dense, ld, ind, li = dense.cpu().numpy(), ld.cpu().numpy(), ind.cpu().numpy(), li.cpu().numpy()
    np.testing.assert_array_equal(dense.view(np.int32), ind.view(np.int32))
    np.testing.assert_array_equal(ld.view(np.int32), li.view(np.int32))
    ref, lse_ref = oracle.latent_attention(F(qa_bits), w.cache, lens, w.scale)
    assert_parity(dense, ref, f"pairs Q={Q} splits={splits}")
    np.testing.assert_allclose(ld, lse_ref, rtol=0, atol=1e-3)


@pytest.mark.parametrize("splits", [0, 2])
def test_pairs_with_empty_visible_sets(splits):
    # cache_len < Q: a query before the cache's first position sees nothing (o_lat NaN, lse
    # -inf, as documented).  Q = 4: length 1 leaves queries 0-2 empty (the pair (3, 2) has one
    # empty member, the pair (1, 0) two), length 3 leaves query 0 empty; every other query must
    # match the oracle on the pass it is the tail of.
    Q, Lmax = 4, 100
    lens = np.array([1, 3, 90], np.int32)
    spec = wl.make_spec(3, Q, Lmax, workload_id=1340)
    w = wl.make_workload(spec)
    w.cache_len[:] = lens
    for b in range(3):
        w.cache[b, lens[b]:] = wl.BF16_NAN
    qa_bits = wl.latent_query_bits(spec)
    qa, c, cl, wv = bf16(qa_bits), bf16(w.cache), i32(lens), bf16(w.w_v)
    o, lse = binding.mla_latent_attn(qa, c, cl, Lmax, w.scale, splits)
    out, lse_f = binding.mla_latent_attn_up_v(qa, c, cl, Lmax, w.scale, wv, num_splits=splits)
    torch.cuda.synchronize()
    o, lse, out, lse_f = o.cpu().numpy(), lse.cpu().numpy(), out.cpu().numpy(), lse_f.cpu().numpy()
    for b, L in enumerate(lens):
        for i in range(Q):
            if L - Q + i + 1 <= 0:
                assert np.isnan(o[b, i]).all() and np.isnan(out[b, i]).all(), (b, i)
                assert np.all(lse[b, i] == -np.inf) and np.all(lse_f[b, i] == -np.inf), (b, i)
        qs = [i for i in range(Q) if L - Q + i + 1 > 0]
        sub_q = F(qa_bits)[b:b + 1, qs[0]:]
        ref, lse_ref = oracle.latent_attention(sub_q, w.cache[b:b + 1], lens[b:b + 1], w.scale)
        assert_parity(o[b:b + 1, qs], ref, f"visible queries of sequence {b}")
        np.testing.assert_allclose(lse[b:b + 1, qs], lse_ref, rtol=0, atol=1e-3)
