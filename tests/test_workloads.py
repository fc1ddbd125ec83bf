"""The seeded input generators: determinism, layout and the structure each workload asks for."""
import numpy as np
import torch

from mla_latent_cache_absorb_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        # exact ties: low 16 bits 0x8000, both parities of the kept bit
                        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40008000], np.uint32)).view(np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_deterministic_and_thread_independent(monkeypatch):
    s = np.random.SeedSequence([1, 2])
    a = wl.normal_bf16(s, 3 * wl.CHUNK + 5)
    monkeypatch.setattr(wl, "_threads", lambda: 1)
    b = wl.normal_bf16(np.random.SeedSequence([1, 2]), 3 * wl.CHUNK + 5)
    np.testing.assert_array_equal(a, b)
    w1 = wl.make_workload("decode_b1_l256")
    w2 = wl.make_workload("decode_b1_l256")
    w3 = wl.make_workload("decode_b1_l256", set_index=1)
    for k in ("q", "cache", "w_k", "w_v"):
        np.testing.assert_array_equal(getattr(w1, k), getattr(w2, k))
        assert not np.array_equal(getattr(w1, k), getattr(w3, k))


def test_shapes_and_distributions():
    w = wl.make_workload("decode_b1_l256")
    assert w.q.shape == (1, 1, 64, 256) and w.q.dtype == np.uint16
    assert w.cache.shape == (1, 256, 512)
    assert w.w_k.shape == (64, 256, 512) and w.w_v.shape == (64, 256, 512)
    f = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for a, std in ((w.cache, 1.0), (w.w_k, np.sqrt(1 / 512)), (w.w_v, np.sqrt(1 / 512))):
        v = f(a)
        assert abs(v.mean()) < 0.02 * std
        assert abs(v.std() / std - 1) < 0.02
    assert w.scale == 1.0 / 16


def test_spikes_exact_count_and_scale():
    spec = wl.make_spec(2, 1, 5000, spike_frac=0.01, spike_scale=8.0, workload_id=3, heads=2)
    w = wl.make_workload(spec)
    base = wl.make_workload(wl.make_spec(2, 1, 5000, workload_id=3, heads=2))
    for b in range(2):
        pos = w.spikes[b]
        assert pos.size == 50 and np.all(np.diff(pos) > 0)
        f = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
        np.testing.assert_array_equal(f(w.cache[b, pos]), f(base.cache[b, pos]) * 8)
        others = np.setdiff1d(np.arange(5000), pos)
        np.testing.assert_array_equal(w.cache[b, others], base.cache[b, others])


def test_ragged_indexed_structure():
    spec = wl.make_spec(4, 4, 3000, min_cache_len=2500, n_index=300, workload_id=4, heads=2)
    w = wl.make_workload(spec)
    assert np.all((w.cache_len >= 2500) & (w.cache_len <= 3000))
    assert w.idx.shape == (4, 4, 304)
    for b in range(4):
        L = int(w.cache_len[b])
        assert np.all(w.cache[b, L:] == wl.BF16_NAN)
        for i in range(4):
            n = int(w.idx_len[b, i])
            assert n == 300 + i + 1
            sel = w.idx[b, i, :n]
            assert np.all(np.diff(sel) > 0)
            assert sel[299] < L - 4                       # drawn from the committed prefix
            np.testing.assert_array_equal(sel[300:], np.arange(L - 4, L - 4 + i + 1))  # causal tail
            assert np.all(w.idx[b, i, n:] == -1)


def test_named_workloads_cover_the_five_cases():
    W = wl.WORKLOADS
    assert (W["decode_b32_l8192"].batch, W["decode_b32_l8192"].q_len, W["decode_b32_l8192"].cache_len) == (32, 1, 8192)
    assert (W["verify_b16_q6_l32768"].batch, W["verify_b16_q6_l32768"].q_len) == (16, 6)
    s = W["decode_b4_l131072_spiked"]
    assert (s.batch, s.cache_len, s.spike_frac, s.spike_scale) == (4, 131072, 0.01, 8.0)
    s = W["indexed_verify_b32_q4_ragged"]
    assert (s.batch, s.q_len, s.min_cache_len, s.cache_len, s.n_index) == (32, 4, 4096, 65536, 2048)


def test_cache_lengths_match_the_workload():
    w = wl.make_workload(wl.make_spec(5, 2, 300, min_cache_len=10, workload_id=77))
    np.testing.assert_array_equal(wl.cache_lengths(w.spec), w.cache_len)
