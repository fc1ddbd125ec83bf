"""GPU parity: the HIP path, called through the C ABI, against the fp64 CPU oracle on the same
seeded inputs.  Bar on fp32 outputs: max|gpu - ref| <= 1e-2 * max|ref| + 1e-3 (per case,
over the whole compared output); selected positions must match exactly (selection probes).
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests import probe_inputs as pi
from tests.gpu_util import DEV, assert_parity, bf16, bits, f32, i32, lse_bound, whole_output_reference

pytestmark = pytest.mark.gpu

F = oracle.bf16_bits_to_f64


def run_path(w, num_splits=0, return_stages=False, two_term=False):
    q, c, wk, wv = bf16(w.q), bf16(w.cache), bf16(w.w_k), bf16(w.w_v)
    cl = i32(w.cache_len)
    Lmax = int(w.cache.shape[1])
    q_abs, q_lo = binding.mla_absorb_q(q, wk, lo=True) if two_term else (binding.mla_absorb_q(q, wk), None)
    if w.idx is None:
        o_lat, lse = binding.mla_latent_attn(q_abs, c, cl, Lmax, w.scale, num_splits, q_abs_lo=q_lo)
    else:
        o_lat, lse = binding.mla_latent_attn_indexed(q_abs, c, cl, i32(w.idx), i32(w.idx_len), Lmax, w.scale,
                                                     num_splits, q_abs_lo=q_lo)
    out = binding.mla_up_v(o_lat, wv)
    torch.cuda.synchronize()
    res = (out.cpu().numpy(), lse.cpu().numpy())
    if return_stages:
        res = res + (bits(q_abs), o_lat.cpu().numpy())
    return res


# ------------------------------------------------------------------ stage: absorb_q
@pytest.mark.parametrize("rows", [1, 4, 33, 128])
def test_absorb_q_matches_definition(rows):
    spec = wl.make_spec(rows, 1, 1, workload_id=200 + rows)
    w = wl.make_workload(spec)
    q_abs = binding.mla_absorb_q(bf16(w.q), bf16(w.w_k))
    torch.cuda.synchronize()
    got_bits = bits(q_abs)
    got = F(got_bits)
    ref = oracle.absorbed_query(w.q, w.w_k)
    # fp32 accumulation then one round-to-nearest-even to bf16: within half a bf16 ulp of the
    # exact value (at most 2^-8 relative), plus fp32 accumulation noise
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    exact = float((got_bits == wl.f32_to_bf16_bits(ref.astype(np.float32))).mean())
    print(f"absorb_q rows={rows}: max err/bound = {float((err / bound).max()):.3f}, "
          f"bit-equal to RNE of the exact value: {exact:.5f}")
    assert (err <= bound).all()
    # only values within fp32 accumulation noise of a rounding midpoint may round the other way
    assert exact > 0.999


def test_absorb_q_prescale_is_exact_power_of_two():
    w = wl.make_workload(wl.make_spec(8, 1, 1, workload_id=210))
    a = binding.mla_absorb_q(bf16(w.q), bf16(w.w_k))
    b = binding.mla_absorb_q(bf16(w.q), bf16(w.w_k), prescale=1.0 / 16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(F(bits(a)) / 16, F(bits(b)))


# ------------------------------------------------------------------ stage: up_v
# rows in passes of 16: 1 (a pass of 8), 32, 37 (a second group of one partial pass), 128, 300
# (groups of ten passes, the last one of twelve rows), 1,100 (sixteen passes a group, the cap)
@pytest.mark.parametrize("rows", [1, 32, 37, 128, 300, 1100])
def test_up_v_matches_definition(rows):
    w = wl.make_workload(wl.make_spec(1, 1, 1, workload_id=220))
    rng = np.random.default_rng(rows)
    o_lat = (rng.standard_normal((rows, 64, 512)) * 0.2).astype(np.float32)
    out = binding.mla_up_v(f32(o_lat), bf16(w.w_v))
    torch.cuda.synchronize()
    ref = oracle.up_project(o_lat.astype(np.float64), w.w_v)
    got = out.cpu().numpy()
    err = float(np.abs(got - ref).max())
    print(f"up_v rows={rows}: max|err| = {err:.3e}, max|ref| = {float(np.abs(ref).max()):.3e}")
    # two bf16 terms keep ~16 bits of o_lat; fp32 accumulation over 512 terms
    assert err <= 1e-4 * float(np.abs(ref).max()) + 1e-6


# ------------------------------------------------------------------ stage: latent attention
LAT_CASES = [
    # B, Q, L, ragged lengths, num_splits
    (1, 1, 1, None, 0),
    (2, 1, 31, None, 0),
    (2, 1, 33, [33, 32], 0),
    (3, 1, 1000, [1000, 517, 64], 0),
    (3, 1, 1000, [1000, 517, 64], 1),
    (3, 1, 1000, [1000, 517, 64], 7),
    (2, 6, 300, [300, 97], 0),
    (2, 6, 300, [300, 97], 1),
    (2, 4, 2100, [2100, 1500], 0),
    (2, 16, 301, [301, 170], 0),    # a 16-position pass; a length bound that is not a whole tile
    (2, 16, 301, [301, 170], 5),
]


@pytest.mark.parametrize("B,Q,L,lens,splits", LAT_CASES)
def test_latent_attn_matches_oracle(B, Q, L, lens, splits):
    spec = wl.make_spec(B, Q, L, workload_id=300 + L + Q)
    w = wl.make_workload(spec)
    if lens is not None:
        w.cache_len[:] = lens
        for b in range(B):
            w.cache[b, lens[b]:] = wl.BF16_NAN
    qa = wl.latent_query_bits(spec)
    o_lat, lse = binding.mla_latent_attn(bf16(qa), bf16(w.cache), i32(w.cache_len), L, w.scale, splits)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.latent_attention(F(qa), w.cache, w.cache_len, w.scale)
    assert_parity(o_lat.cpu().numpy(), ref, f"o_lat B{B} Q{Q} L{L} s{splits}")
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=1e-3)


def test_indexed_latent_attn_matches_oracle():
    spec = wl.make_spec(3, 4, 3000, min_cache_len=2000, n_index=500, workload_id=330)
    w = wl.make_workload(spec)
    qa = wl.latent_query_bits(spec)
    for splits in (0, 1, 5):
        o_lat, lse = binding.mla_latent_attn_indexed(bf16(qa), bf16(w.cache), i32(w.cache_len), i32(w.idx),
                                                     i32(w.idx_len), 3000, w.scale, splits)
        torch.cuda.synchronize()
        ref, lse_ref = oracle.latent_attention(F(qa), w.cache, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len)
        assert_parity(o_lat.cpu().numpy(), ref, f"indexed o_lat s{splits}")
        np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=1e-3)


# ------------------------------------------------------------------ many splits
def test_many_splits_more_workgroups_than_cus():
    # more split workgroups than CUs (several rounds of workgroups), ragged lengths
    B, L = 48, 1024
    spec = wl.make_spec(B, 1, L, min_cache_len=200, workload_id=620)
    w = wl.make_workload(spec)
    qa = bf16(wl.latent_query_bits(spec))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = 8
    assert B * splits > cus
    o, lse = binding.mla_latent_attn(qa, bf16(w.cache), i32(w.cache_len), L, w.scale, splits)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.latent_attention(F(bits(qa)), w.cache, w.cache_len, w.scale)
    assert_parity(o.cpu().numpy(), ref, "separate merge")
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=1e-3)


def test_maximum_split_count():
    # 1,024 splits of one 32-position tile each over a 32,768-position cache: the largest split
    # count, the wide merge in sixteen rounds of eight groups; the fused call gives the same bits
    spec = wl.make_spec(1, 1, 32768, workload_id=630)
    w = wl.make_workload(spec)
    assert binding.mla_latent_attn_num_splits(1, 1, 64, 32768, 5000) == 1024
    qa = bf16(wl.latent_query_bits(spec))
    c, cl, wv = bf16(w.cache), i32(w.cache_len), bf16(w.w_v)
    print("1024 splits", flush=True)
    o, lse = binding.mla_latent_attn(qa, c, cl, 32768, w.scale, 1024)
    out_s = binding.mla_up_v(o, wv)
    out_f, lse_f = binding.mla_latent_attn_up_v(qa, c, cl, 32768, w.scale, wv, num_splits=1024)
    torch.cuda.synchronize()
    assert torch.equal(out_f.view(torch.int32), out_s.view(torch.int32))
    assert torch.equal(lse_f.view(torch.int32), lse.view(torch.int32))
    hs = [0, 21, 63]
    ref, lse_ref = oracle.latent_attention(F(bits(qa)), w.cache, w.cache_len, w.scale, heads=hs)
    assert_parity(o.cpu().numpy()[:, :, hs], ref, "1024 splits")
    np.testing.assert_allclose(lse.cpu().numpy()[:, :, hs], lse_ref, rtol=0, atol=1e-3)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_empty_visible_sets(splits):
    # cache_len < Q: a query before the cache's first position sees nothing and gets o_lat = NaN,
    # lse = -inf, out = NaN, as documented; every other query of the call is unaffected.
    # Sequence 0 (length 1): queries 0, 1 empty, query 2 sees position 0.  Sequence 1 (length 2):
    # query 0 empty, queries 1 and 2 see 0 and 0..1.  Sequence 2 (length 90): every query normal.
    Q, Lmax = 3, 100
    spec = wl.make_spec(3, Q, Lmax, workload_id=640)
    w = wl.make_workload(spec)
    lens = np.array([1, 2, 90], np.int32)
    w.cache_len[:] = lens
    for b in range(3):
        w.cache[b, lens[b]:] = wl.BF16_NAN
    qa_bits = wl.latent_query_bits(spec)
    qa, c, cl, wv = bf16(qa_bits), bf16(w.cache), i32(lens), bf16(w.w_v)
    o, lse = binding.mla_latent_attn(qa, c, cl, Lmax, w.scale, splits)
    out, lse_f = binding.mla_latent_attn_up_v(qa, c, cl, Lmax, w.scale, wv, num_splits=splits)
    torch.cuda.synchronize()
    o, lse, out, lse_f = o.cpu().numpy(), lse.cpu().numpy(), out.cpu().numpy(), lse_f.cpu().numpy()
    empty = [(0, 0), (0, 1), (1, 0)]
    for b, i in empty:
        assert np.isnan(o[b, i]).all() and np.isnan(out[b, i]).all(), (b, i)
        assert np.all(lse[b, i] == -np.inf) and np.all(lse_f[b, i] == -np.inf), (b, i)
    # the visible queries, each against the oracle on the pass it is the tail of
    for b, qs in ((0, [2]), (1, [1, 2]), (2, [0, 1, 2])):
        n = len(qs)
        sub_q = F(qa_bits)[b:b + 1, qs[0]:]
        ref, lse_ref = oracle.latent_attention(sub_q, w.cache[b:b + 1], lens[b:b + 1], w.scale)
        assert np.isfinite(o[b, qs]).all() and np.isfinite(out[b, qs]).all()
        assert_parity(o[b:b + 1, qs], ref, f"visible queries of sequence {b}")
        np.testing.assert_allclose(lse[b:b + 1, qs], lse_ref, rtol=0, atol=1e-3)
        assert n == ref.shape[1]


# ------------------------------------------------------------------ q_len sweep
# Draft depths 0..7 (one to eight query positions per pass): the query-to-position mapping and
# the causal tail of the last tile for every depth, dense and indexed, ragged lengths, through
# the whole path (absorb, attention, up-projection).
@pytest.mark.parametrize("Q", [1, 2, 3, 4, 5, 6, 7, 8])
def test_q_len_sweep_whole_path(Q):
    spec = wl.make_spec(3, Q, 203, min_cache_len=Q, workload_id=500 + Q)
    w = wl.make_workload(spec)
    out, lse = run_path(w)
    ref, lse_ref = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale)
    assert_parity(out, ref, f"dense Q{Q} out")
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-2)
    spec_i = wl.make_spec(2, Q, 300, min_cache_len=100, n_index=40, workload_id=520 + Q)
    wi = wl.make_workload(spec_i)
    out, lse = run_path(wi)
    ref, lse_ref = oracle.mla_reference(wi.q, wi.cache, wi.w_k, wi.w_v, wi.cache_len, wi.scale, idx=wi.idx,
                                        idx_len=wi.idx_len)
    assert_parity(out, ref, f"indexed Q{Q} out")
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-2)


# ------------------------------------------------------------------ whole path, small
def test_decode_b1_l256_whole_output():
    w = wl.make_workload("decode_b1_l256")
    out, lse, q_abs, o_lat = run_path(w, return_stages=True)
    ref, lse_ref = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale)
    assert_parity(out, ref, "decode_b1_l256 out")
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-2)


@pytest.mark.parametrize("B,Q,L", [(2, 6, 129), (3, 2, 40), (1, 5, 5)])
def test_verify_small_whole_output(B, Q, L):
    w = wl.make_workload(wl.make_spec(B, Q, L, workload_id=400 + L))
    out, lse = run_path(w)
    ref, lse_ref = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale)
    assert_parity(out, ref, f"verify B{B} Q{Q} L{L} out")
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-2)


# ------------------------------------------------------------------ whole path, full sizes
# The spiked workload runs with the absorbed query in two bf16 terms: with one, the rounding of q~
# alone moves its worst row past the bar (the attention call itself matches the oracle given the
# same rounded q~ at every row: tests/test_gpu_full_size.py).
FULL = [
    ("decode_b32_l8192", [0, 31], None, [0, 17, 63], False),
    ("verify_b16_q6_l32768", [0, 15], None, [5, 40], False),
    ("decode_b4_l131072_spiked", [1, 3], None, [0, 33], True),
    ("indexed_verify_b32_q4_ragged", [0, 19], None, [2, 61], False),
]


@pytest.mark.parametrize("name,bs,qs,hs,two_term", FULL)
def test_full_size_sampled(name, bs, qs, hs, two_term):
    print(f"full-size case {name}{' (two-term query)' if two_term else ''}: generating inputs", flush=True)
    w = wl.make_workload(name)
    out, lse = run_path(w, two_term=two_term)
    print(f"{name}: GPU done, oracle on batches {bs} heads {hs}", flush=True)
    ref, lse_ref = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, idx=w.idx,
                                        idx_len=w.idx_len, batches=bs, queries=qs, heads=hs)
    qs_all = list(range(w.q.shape[1]))
    got = out[np.ix_(bs, qs_all, hs)]
    # every row against the oracle's absorbed fp64 form; the sampled rows above also against its
    # expanded form, the bar relative to the largest value of the whole output
    ref_all = whole_output_reference(w)
    assert_parity(out, ref_all, f"{name} out, every row")
    assert_parity(got, ref, f"{name} sampled out", ref_max=float(np.abs(ref_all).max()))
    lerr = np.abs(lse[np.ix_(bs, qs_all, hs)] - lse_ref)
    lbar = lse_bound(w, bs, qs_all, hs)
    print(f"{name}: max|lse err| = {float(lerr.max()):.3e}, max err/bound = {float((lerr / lbar).max()):.3f}")
    assert (lerr <= lbar).all()
    assert np.isfinite(out).all()


# ------------------------------------------------------------------ selection probes
# Position-coded latents and a query per head that counts the visible positions with one code bit
# set; the counts are read from lse (tests/probe_inputs.py), which the library computes in fp32
# from the running maxima and sums only.
def probe_query(B, Q):
    return bf16(np.ascontiguousarray(np.broadcast_to(pi.lse_probe_query(), (B, Q, 64, 512))))


def assert_probe_counts(lse_row, positions, what):
    got, dist = pi.decoded_lse_counts(lse_row)
    want = pi.expected_lse_counts(positions)
    assert dist < 0.3, f"{what}: lse {dist:.3f} from an integer count"
    np.testing.assert_array_equal(got, want, err_msg=what)


def _probe_dense(B, Q, L_max, lens, splits):
    cache = pi.coded_cache(B, L_max, 512, np.array(lens))
    o_lat, lse = binding.mla_latent_attn(probe_query(B, Q), bf16(cache), i32(lens), L_max, 1.0 / 16, splits)
    torch.cuda.synchronize()
    return o_lat.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_probe_dense_selects_exact_causal_sets(splits):
    B, Q, L_max = 3, 6, 700
    lens = [700, 641, 65]
    o_lat, lse = _probe_dense(B, Q, L_max, lens, splits)
    assert np.isfinite(o_lat).all(), "a row past cache_len was read (NaN poison)"
    for b in range(B):
        for i in range(Q):
            assert_probe_counts(lse[b, i], oracle.dense_visible_positions(lens[b], Q, i), f"b{b} i{i}")


def test_probe_indexed_reads_only_listed_slots():
    B, Q, L_max, K = 2, 4, 900, 300
    lens = np.array([900, 513], np.int32)
    rng = np.random.default_rng(5)
    idx = np.zeros((B, Q, K), np.int32)
    idx_len = np.zeros((B, Q), np.int32)
    sets = {}
    for b in range(B):
        for i in range(Q):
            t = lens[b] - Q + i
            n = int(rng.integers(1, K + 1))
            sel = np.sort(rng.choice(t + 1, size=min(n, t + 1), replace=False)).astype(np.int32)
            idx[b, i, :sel.size] = sel
            idx_len[b, i] = sel.size
            # slots past idx_len name valid positions outside the set: reading them changes counts
            rest = np.setdiff1d(np.arange(t + 1), sel)[: K - sel.size]
            idx[b, i, sel.size:sel.size + rest.size] = rest
            sets[(b, i)] = sel
    cache = pi.coded_cache(B, L_max, 512, lens)
    q_abs = probe_query(B, Q)
    for splits in (0, 1, 4):
        o_lat, lse = binding.mla_latent_attn_indexed(q_abs, bf16(cache), i32(lens), i32(idx), i32(idx_len), L_max,
                                                     1.0 / 16, splits)
        torch.cuda.synchronize()
        o_lat, lse = o_lat.cpu().numpy(), lse.cpu().numpy()
        assert np.isfinite(o_lat).all()
        for (b, i), sel in sets.items():
            assert_probe_counts(lse[b, i], sel, f"b{b} i{i} s{splits}")


def test_spike_at_first_masked_position_does_not_leak():
    # query 0 of a 6-position pass must not see position L-6+1 (query 1 does).  That row holds a
    # spike aligned with query 0's absorbed query at head 7, so a causal bound one too wide
    # would make it dominate query 0's output there.
    spec = wl.make_spec(1, 6, 500, workload_id=450)
    w = wl.make_workload(spec)
    qa = wl.latent_query_bits(spec)
    qt = F(qa[0, 0, 7])
    spike = wl.f32_to_bf16_bits((qt / np.linalg.norm(qt) * 300.0).astype(np.float32))
    w.cache[0, 500 - 6 + 1] = spike
    o_lat, lse = binding.mla_latent_attn(bf16(qa), bf16(w.cache), i32(w.cache_len), 500, w.scale, 0)
    torch.cuda.synchronize()
    ref, lse_ref = oracle.latent_attention(F(qa), w.cache, w.cache_len, w.scale)
    o = o_lat.cpu().numpy()
    assert_parity(o[0, 0], ref[0, 0], "query 0 (spike masked)")
    assert_parity(o[0, 1], ref[0, 1], "query 1 (spike visible)")
    # the probe can fail: with the spike visible, query 0's head 7 would be the spike itself
    leaked = np.abs(F(spike) - o[0, 0, 7]).max()
    assert leaked > 100 * (1e-2 * np.abs(ref[0, 0]).max() + 1e-3)


# ------------------------------------------------------------------ invariances
def test_split_count_invariance_and_determinism():
    spec = wl.make_spec(2, 2, 4000, workload_id=460)
    w = wl.make_workload(spec)
    qa = bf16(wl.latent_query_bits(spec))
    c, cl = bf16(w.cache), i32(w.cache_len)
    outs = {}
    for s in (1, 2, 9, 0):
        outs[s] = binding.mla_latent_attn(qa, c, cl, 4000, w.scale, s)[0].cpu().numpy()
    ref = outs[1]
    for s, o in outs.items():
        assert_parity(o, ref, f"splits {s} vs 1")
    again = binding.mla_latent_attn(qa, c, cl, 4000, w.scale, 9)[0].cpu().numpy()
    np.testing.assert_array_equal(again, outs[9])


@pytest.mark.parametrize("Q", [1, 3])
def test_indexed_with_full_causal_set_equals_dense(Q):
    # listing every causal position reproduces the dense call bit for bit: both calls run the
    # same schedule (same splits, tiles and arithmetic order); only where rows come from differs
    B, L = 2, 700
    spec = wl.make_spec(B, Q, L, workload_id=470)
    w = wl.make_workload(spec)
    idx = np.full((B, Q, L), -1, np.int32)
    idx_len = np.zeros((B, Q), np.int32)
    for b in range(B):
        for i in range(Q):
            n = L - Q + i + 1
            idx[b, i, :n] = np.arange(n)
            idx_len[b, i] = n
    qa = bf16(wl.latent_query_bits(spec))
    dense, ld = binding.mla_latent_attn(qa, bf16(w.cache), i32(w.cache_len), L, w.scale, 4)
    ind, li = binding.mla_latent_attn_indexed(qa, bf16(w.cache), i32(w.cache_len), i32(idx), i32(idx_len), L,
                                              w.scale, 4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ind.cpu().numpy(), dense.cpu().numpy())
    np.testing.assert_array_equal(li.cpu().numpy(), ld.cpu().numpy())


def test_rollback_equals_never_generated():
    # verify 6 positions at L, reject after draft 2: the cache is truncated to L - 6 + 3 and the
    # next decode must equal a run on a cache that never held the rejected rows
    spec = wl.make_spec(2, 1, 1200, workload_id=480)
    w = wl.make_workload(spec)
    qa = bf16(wl.latent_query_bits(spec))
    keep = np.array([1200 - 6 + 3, 1200 - 6 + 1], np.int32)
    a, la = binding.mla_latent_attn(qa, bf16(w.cache), i32(keep), 1200, w.scale, 0)
    fresh = w.cache.copy()
    for b in range(2):
        fresh[b, keep[b]:] = wl.BF16_NAN
    b_, lb = binding.mla_latent_attn(qa, bf16(fresh), i32(keep), 1200, w.scale, 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b_.cpu().numpy())
    np.testing.assert_array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_cache_batch_stride_view():
    # a cache allocated with more rows than max_cache_len, passed as a view
    spec = wl.make_spec(2, 1, 300, workload_id=490)
    w = wl.make_workload(spec, l_max=450)
    qa = wl.latent_query_bits(spec)
    big = bf16(w.cache)
    o_lat, lse = binding.mla_latent_attn(bf16(qa), big[:, :300], i32(w.cache_len), 300, w.scale, 0)
    torch.cuda.synchronize()
    ref, _ = oracle.latent_attention(F(qa), w.cache, w.cache_len, w.scale)
    assert_parity(o_lat.cpu().numpy(), ref, "strided cache")


# ------------------------------------------------------------------ errors leave outputs untouched
def test_errors_write_nothing():
    spec = wl.make_spec(1, 1, 64, workload_id=495)
    w = wl.make_workload(spec)
    qa = bf16(wl.latent_query_bits(spec))
    o = torch.full((1, 1, 64, 512), 7.0, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(binding.MlaError) as e:
        binding.mla_latent_attn(qa, bf16(w.cache), i32(w.cache_len), 64, w.scale, 2, o_lat=o, workspace=small)
    assert e.value.status == binding.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
    L = binding.lib()
    rc = L.mla_latent_attn(binding._ptr(qa), None, binding._ptr(bf16(w.cache)), 64 * 512,
                           binding._ptr(i32(w.cache_len)), 1, 1, 64, 256, 64, w.scale, 0, binding._ptr(o), None, None,
                           0, None)
    assert rc == binding.MLA_ERR_SHAPE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
