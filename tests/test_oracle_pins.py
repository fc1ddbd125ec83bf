"""Pins for the CPU oracle: checks against things other than the oracle itself.

* the page's printed cache arithmetic (golden fixture, Module 05 section 2);
* brute-force scalar loops on tiny inputs;
* a library routine: torch's fp64 scaled_dot_product_attention on expanded K, V;
* the absorption identity of Module 05 section 3 / colibri "MLA is absorbed" (scores AND outputs);
* closed-form special cases (single position, zero query, equal latents, a dominant spike,
  permutation inside the visible set, indexed-with-the-full-set, truncation);
* planted mistakes in the oracle (on the CPU) that the pins above must catch.
"""
import json
import math
import os
import struct

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import mla_oracle
from mla_latent_cache_absorb_amd import workloads as wl
from tests import probe_inputs as pi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_workload(B=2, Q=3, L=6, H=2, D=3, R=4, seed=7, indexed=False, n_index=0):
    spec = wl.make_spec(B, Q, L, heads=H, head_dim=D, latent=R, workload_id=seed, n_index=n_index,
                        scale=0.37)
    return wl.make_workload(spec)


# ---------------------------------------------------------------- golden: page numbers
def test_cache_arithmetic_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "cache_bytes_per_token.json")))
    exp_b, lat_b = oracle.cache_bytes_per_token(g["heads"], g["head_dim"], g["latent"], g["bytes_per_value"])
    assert exp_b == g["expanded_bytes_per_token_per_layer"] == 65536
    assert lat_b == g["latent_bytes_per_token_per_layer"] == 1024
    assert exp_b // lat_b == g["ratio"] == 64
    # the workloads use the checkpoint's dimensions
    assert (wl.HEADS, wl.HEAD_DIM, wl.LATENT) == (g["heads"], g["head_dim"], g["latent"])
    # a latent cache row is exactly 1,024 bytes of bf16
    w = wl.make_workload("decode_b1_l256")
    assert w.cache.strides[1] == lat_b


# ---------------------------------------------------------------- brute force
def _bf(bits):
    return struct.unpack(">f", struct.pack(">I", int(bits) << 16))[0]


def brute_force(w, dense=True):
    """Scalar loops over the definition: k = U^K c, v = U^V c, softmax of scale*q.k over j <= t."""
    B, Q, H, D = w.q.shape
    R = w.cache.shape[2]
    out = np.zeros((B, Q, H, D))
    lse = np.zeros((B, Q, H))
    for b in range(B):
        L = int(w.cache_len[b])
        for i in range(Q):
            t = L - Q + i
            if dense:
                vis = [j for j in range(L) if j <= t]
            else:
                vis = [int(x) for x in w.idx[b, i, : w.idx_len[b, i]]]
            for h in range(H):
                s, vs = [], []
                for j in vis:
                    c = [_bf(w.cache[b, j, r]) for r in range(R)]
                    k = [sum(_bf(w.w_k[h, d, r]) * c[r] for r in range(R)) for d in range(D)]
                    v = [sum(_bf(w.w_v[h, d, r]) * c[r] for r in range(R)) for d in range(D)]
                    s.append(w.scale * sum(_bf(w.q[b, i, h, d]) * k[d] for d in range(D)))
                    vs.append(v)
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for d in range(D):
                    out[b, i, h, d] = sum(e[n] / z * vs[n][d] for n in range(len(vis)))
                lse[b, i, h] = m + math.log(z)
    return out, lse


def test_brute_force_dense_tiny():
    w = tiny_workload()
    w.cache_len[:] = [6, 4]
    ref, lse_ref = brute_force(w)
    out, lse = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-14)


def _tiny_indexed():
    w = tiny_workload(B=2, Q=2, L=6)
    K = 5
    w.idx = np.full((2, 2, K), -1, np.int32)
    w.idx_len = np.zeros((2, 2), np.int32)
    sets = {(0, 0): [0, 2, 4], (0, 1): [1, 5], (1, 0): [3], (1, 1): [0, 1, 2, 4, 5]}
    for (b, i), s in sets.items():
        w.idx[b, i, : len(s)] = s
        w.idx_len[b, i] = len(s)
    return w


def test_brute_force_indexed_tiny():
    w = _tiny_indexed()
    ref, lse_ref = brute_force(w, dense=False)
    out, lse = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- library routine
def sdpa_reference(w, dense=True):
    """torch fp64 scaled_dot_product_attention on expanded K, V with an explicit boolean mask."""
    f = lambda a: torch.from_numpy(oracle.bf16_bits_to_f64(a))
    q, c, wk, wv = f(w.q), f(w.cache), f(w.w_k), f(w.w_v)
    B, Q, H, D = q.shape
    L = c.shape[1]
    c = torch.nan_to_num(c, nan=0.0)  # padded rows are masked out below
    k = torch.einsum("blr,hdr->bhld", c, wk)
    v = torch.einsum("blr,hdr->bhld", c, wv)
    mask = torch.zeros(B, 1, Q, L, dtype=torch.bool)
    for b in range(B):
        for i in range(Q):
            if dense:
                mask[b, 0, i, : int(w.cache_len[b]) - Q + i + 1] = True
            else:
                mask[b, 0, i, torch.from_numpy(w.idx[b, i, : w.idx_len[b, i]].astype(np.int64))] = True
    out = torch.nn.functional.scaled_dot_product_attention(q.permute(0, 2, 1, 3), k, v, attn_mask=mask,
                                                           scale=w.scale)
    s = torch.einsum("bqhd,bhld->bhql", q, k) * w.scale
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


@pytest.mark.parametrize("B,Q,L,H", [(1, 1, 256, 4), (2, 6, 70, 3), (3, 4, 33, 2)])
def test_matches_torch_sdpa_dense(B, Q, L, H):
    spec = wl.make_spec(B, Q, L, heads=H, workload_id=11)
    w = wl.make_workload(spec)
    if B > 1:
        w.cache_len[1:] = np.arange(L - B + 1, L)[: B - 1]  # ragged, NaN past the end
        for b in range(1, B):
            w.cache[b, w.cache_len[b]:] = wl.BF16_NAN
    ref, lse_ref = sdpa_reference(w)
    out, lse = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_matches_torch_sdpa_indexed():
    spec = wl.make_spec(2, 4, 300, heads=3, n_index=40, min_cache_len=200, workload_id=12)
    w = wl.make_workload(spec)
    ref, lse_ref = sdpa_reference(w, dense=False)
    out, lse = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- absorption identity
def absorbed_by_identity(w, dense=True):
    """Absorbed form, written from the identity (independently of the oracle's code):
    q~ = W_k^T q, s_j = scale q~.c_j, out = W_v (sum_j a_j c_j); scipy's logsumexp."""
    f = oracle.bf16_bits_to_f64
    q, c, wk, wv = f(w.q), f(w.cache), f(w.w_k), f(w.w_v)
    B, Q, H, D = q.shape
    qt = np.einsum("bqhd,hdr->bqhr", q, wk)
    out = np.zeros((B, Q, H, D))
    lse = np.zeros((B, Q, H))
    scores = {}
    for b in range(B):
        for i in range(Q):
            if dense:
                pos = np.arange(int(w.cache_len[b]) - Q + i + 1)
            else:
                pos = w.idx[b, i, : w.idx_len[b, i]].astype(np.int64)
            cb = c[b, pos]
            s = w.scale * np.einsum("hr,jr->hj", qt[b, i], cb)
            scores[(b, i)] = (pos, s)
            lz = scipy.special.logsumexp(s, axis=1)
            a = np.exp(s - lz[:, None])
            olat = a @ cb
            out[b, i] = np.einsum("hdr,hr->hd", wv, olat)
            lse[b, i] = lz
    return out, lse, scores


@pytest.mark.parametrize("indexed", [False, True])
def test_absorption_identity_outputs_and_scores(indexed):
    if indexed:
        spec = wl.make_spec(2, 3, 500, heads=4, n_index=64, min_cache_len=300, workload_id=13)
    else:
        spec = wl.make_spec(2, 3, 400, heads=4, workload_id=14)
    w = wl.make_workload(spec)
    out_a, lse_a, scores = absorbed_by_identity(w, dense=not indexed)
    kw = dict(idx=w.idx, idx_len=w.idx_len) if indexed else {}
    out, lse = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, **kw)
    np.testing.assert_allclose(out, out_a, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, lse_a, rtol=1e-12, atol=1e-13)
    # the scores themselves must be equal, not merely proportional (Module 05 section 3)
    for (b, i), (pos, s) in scores.items():
        for h in range(spec.heads):
            se = oracle.expanded_scores(w.q, w.cache, w.w_k, w.scale, b, i, h, pos)
            np.testing.assert_allclose(se, s[h], rtol=1e-11, atol=1e-13)


def test_absorbed_stages_compose_to_reference():
    spec = wl.make_spec(2, 2, 300, heads=4, workload_id=15)
    w = wl.make_workload(spec)
    qt = oracle.absorbed_query(w.q, w.w_k)
    olat, lse_l = oracle.latent_attention(qt, w.cache, w.cache_len, w.scale)
    out_s = oracle.up_project(olat, w.w_v)
    out, lse = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale)
    np.testing.assert_allclose(out_s, out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse_l, lse, rtol=1e-12)
    # absorbed query against an einsum over the stored layout
    np.testing.assert_allclose(qt, np.einsum("bqhd,hdr->bqhr", oracle.bf16_bits_to_f64(w.q),
                                             oracle.bf16_bits_to_f64(w.w_k)), rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- special cases
def _ref(w, **kw):
    return oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, **kw)


def test_single_position_outputs_its_value():
    spec = wl.make_spec(1, 1, 1, heads=3, workload_id=16)
    w = wl.make_workload(spec)
    out, lse = _ref(w)
    c0 = oracle.bf16_bits_to_f64(w.cache[0, 0])
    for h in range(3):
        vh = oracle.bf16_bits_to_f64(w.w_v[h]) @ c0
        np.testing.assert_allclose(out[0, 0, h], vh, rtol=1e-15, atol=1e-15)
        s = w.scale * (oracle.bf16_bits_to_f64(w.q[0, 0, h]) @ (oracle.bf16_bits_to_f64(w.w_k[h]) @ c0))
        assert abs(lse[0, 0, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_zero_query_is_uniform_average():
    spec = wl.make_spec(2, 3, 50, heads=2, workload_id=17)
    w = wl.make_workload(spec)
    w.q[:] = 0
    out, lse = _ref(w)
    for b in range(2):
        for i in range(3):
            n = 50 - 3 + i + 1
            mean_c = oracle.bf16_bits_to_f64(w.cache[b, :n]).mean(axis=0)
            for h in range(2):
                np.testing.assert_allclose(out[b, i, h], oracle.bf16_bits_to_f64(w.w_v[h]) @ mean_c, rtol=1e-12, atol=1e-14)
                assert abs(lse[b, i, h] - math.log(n)) < 1e-12


def test_equal_latents_give_that_value():
    spec = wl.make_spec(1, 2, 40, heads=2, workload_id=18)
    w = wl.make_workload(spec)
    w.cache[0, :] = w.cache[0, 7]
    out, lse = _ref(w)
    c = oracle.bf16_bits_to_f64(w.cache[0, 7])
    for i in range(2):
        for h in range(2):
            np.testing.assert_allclose(out[0, i, h], oracle.bf16_bits_to_f64(w.w_v[h]) @ c, rtol=1e-12, atol=1e-14)


def test_dominant_spike_selects_its_value():
    spec = wl.make_spec(1, 1, 64, heads=1, workload_id=19)
    w = wl.make_workload(spec)
    f = oracle.bf16_bits_to_f64
    # latent aligned with the absorbed query, scaled so its score dominates every other by > 60
    qt = f(w.q[0, 0, 0]) @ f(w.w_k[0])
    spike = wl.f32_to_bf16_bits((qt / np.linalg.norm(qt) * 40.0).astype(np.float32))
    w.cache[0, 23] = spike
    out, _ = _ref(w)
    s = oracle.expanded_scores(w.q, w.cache, w.w_k, w.scale, 0, 0, 0, np.arange(64))
    gap = s[23] - np.delete(s, 23).max()
    assert gap > 30
    np.testing.assert_allclose(out[0, 0, 0], f(w.w_v[0]) @ f(spike), rtol=1e-9, atol=1e-12)


def test_permutation_inside_visible_set_leaves_output_unchanged():
    # NoPE: order enters only through the mask (Module 05 section 4)
    spec = wl.make_spec(1, 1, 80, heads=3, workload_id=20)
    w = wl.make_workload(spec)
    out, lse = _ref(w)
    perm = np.random.default_rng(0).permutation(80)
    w.cache[0] = w.cache[0, perm]
    out2, lse2 = _ref(w)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


def test_indexed_with_full_causal_set_equals_dense():
    spec = wl.make_spec(2, 3, 60, heads=2, workload_id=21)
    w = wl.make_workload(spec)
    K = 60
    idx = np.full((2, 3, K), -1, np.int32)
    idx_len = np.zeros((2, 3), np.int32)
    for b in range(2):
        for i in range(3):
            n = 60 - 3 + i + 1
            idx[b, i, :n] = np.arange(n)
            idx_len[b, i] = n
    out_d, lse_d = _ref(w)
    out_i, lse_i = _ref(w, idx=idx, idx_len=idx_len)
    np.testing.assert_array_equal(out_i, out_d)
    np.testing.assert_array_equal(lse_i, lse_d)


def test_truncated_cache_equals_never_generated_run():
    # rollback of the latent cache is truncation by position (Module 08 section 3)
    spec = wl.make_spec(1, 1, 100, heads=2, workload_id=22)
    w = wl.make_workload(spec)
    w_trunc_len = np.array([73], np.int32)
    out_t, lse_t = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w_trunc_len, w.scale)
    fresh = w.cache.copy()
    fresh[0, 73:] = wl.BF16_NAN  # the rejected rows were never written
    out_f, lse_f = oracle.mla_reference(w.q, fresh, w.w_k, w.w_v, w_trunc_len, w.scale)
    np.testing.assert_array_equal(out_t, out_f)
    np.testing.assert_array_equal(lse_t, lse_f)
    assert np.isfinite(out_t).all()


def test_visible_set_rules():
    assert list(oracle.dense_visible_positions(10, 3, 0)) == list(range(8))
    assert list(oracle.dense_visible_positions(10, 3, 2)) == list(range(10))
    with pytest.raises(ValueError):
        oracle.indexed_visible_positions(np.array([3, 2]), 2, 10, 1, 0)   # unsorted
    with pytest.raises(ValueError):
        oracle.indexed_visible_positions(np.array([3, 9]), 2, 10, 2, 0)   # 9 > position 8
    with pytest.raises(ValueError):
        oracle.indexed_visible_positions(np.array([3, 3]), 2, 10, 1, 0)   # duplicate


# ---------------------------------------------------------------- selection probe (CPU side)
def _probe_case(B=2, Q=6, L=300, H=2):
    cache_len = np.array([L, L - 37][:B], np.int32)
    cache = pi.coded_cache(B, L, 512, cache_len)
    q_abs = np.zeros((B, Q, H, 512))
    return cache, cache_len, q_abs


def test_probe_recovers_selected_sets_exactly():
    cache, cache_len, q_abs = _probe_case()
    olat, lse = oracle.latent_attention(q_abs, cache, cache_len, 1.0 / 16)
    for b in range(2):
        for i in range(6):
            expect = pi.expected_counts(oracle.dense_visible_positions(int(cache_len[b]), 6, i))
            got, n = pi.decoded_counts(olat[b, i, 0], lse[b, i, 0])
            assert n == expect[-1]
            np.testing.assert_array_equal(got, expect)


def _lse_probe_ok(lse, cache_len, Q, batches):
    """Whether the log-sum-exp form of the probe recovers every query's exact causal counts."""
    ok = True
    for b in batches:
        for i in range(Q):
            expect = pi.expected_lse_counts(np.arange(int(cache_len[b]) - Q + i + 1))
            got, dist = pi.decoded_lse_counts(lse[b, i])
            ok &= bool(np.array_equal(got, expect)) and dist < 0.01
    return ok


def test_lse_probe_recovers_selected_sets_exactly():
    # the probe's log-sum-exp form (a query per head that scores 0 on positions with one code bit
    # set and -K elsewhere) on the oracle: every head's lse gives its count exactly
    cache, cache_len, _ = _probe_case()
    q_abs = np.broadcast_to(oracle.bf16_bits_to_f64(pi.lse_probe_query()), (2, 6, 64, 512))
    _, lse = oracle.latent_attention(q_abs, cache, cache_len, 1.0 / 16)
    assert _lse_probe_ok(lse, cache_len, 6, range(2))
    # and for an indexed set
    sel = np.array([3, 17, 64, 65, 200, 250], np.int64)
    idx = np.full((2, 6, 8), -1, np.int32)
    idx_len = np.ones((2, 6), np.int32)
    idx[:, :, 0] = 0
    idx[0, 5, :6] = sel
    idx_len[0, 5] = 6
    _, lse = oracle.latent_attention(q_abs, cache, cache_len, 1.0 / 16, idx=idx, idx_len=idx_len)
    got, _ = pi.decoded_lse_counts(lse[0, 5])
    np.testing.assert_array_equal(got, pi.expected_lse_counts(sel))


# ---------------------------------------------------------------- planted mistakes
MISTAKES = {
    "causal_bound_plus_one": ("dense_visible_positions",
                              lambda orig: (lambda L, Q, i: np.arange(0, L - Q + i + 2 if L - Q + i + 2 <= L else L - Q + i + 1))),
    "causal_bound_minus_one": ("dense_visible_positions",
                               lambda orig: (lambda L, Q, i: np.arange(0, max(1, L - Q + i)))),
    "key_dims_permuted": ("expand_keys", lambda orig: (lambda c, w: orig(c, w)[:, ::-1])),
    "transposed_weights": ("expand_values", lambda orig: (lambda c, w: c @ w)),
    "scale_dropped": ("softmax_attention", lambda orig: (lambda q, k, v, s: orig(q, k, v, 1.0))),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, make = MISTAKES[name]
    orig = getattr(mla_oracle, attr)
    monkeypatch.setattr(mla_oracle, attr, make(orig))
    # square weights (D == R) so that a transposition still runs
    w = tiny_workload(B=1, Q=3, L=6, H=2, D=4, R=4)
    caught = False
    try:
        ref, lse_ref = brute_force(w)
        out, lse = mla_oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale)
        caught = not (np.allclose(out, ref, rtol=1e-9, atol=1e-12) and np.allclose(lse, lse_ref, rtol=1e-9))
    except (ValueError, IndexError):
        caught = True
    if name.startswith("causal"):
        # the selection probe must see it too
        cache, cache_len, q_abs = _probe_case(B=1, Q=3, L=64)
        olat, lse = mla_oracle.latent_attention(q_abs, cache, cache_len, 1.0 / 16)
        probe_ok = True
        for i in range(3):
            expect = pi.expected_counts(np.arange(64 - 3 + i + 1))
            got, n = pi.decoded_counts(olat[0, i, 0], lse[0, i, 0])
            probe_ok &= bool(np.array_equal(got, expect))
        assert not probe_ok, "selection probe missed a shifted causal bound"
        # and so must its log-sum-exp form
        q_lse = np.broadcast_to(oracle.bf16_bits_to_f64(pi.lse_probe_query()), (1, 3, 64, 512))
        _, lse = mla_oracle.latent_attention(q_lse, cache, cache_len, 1.0 / 16)
        assert not _lse_probe_ok(lse, cache_len, 3, [0]), "log-sum-exp probe missed a shifted causal bound"
    assert caught, f"pins missed planted mistake {name}"
