"""Pins of the naive-form stage oracle (CPU only).

Page "Module 05 -- MLA: Compressing Per-Token History", section 5: the naive form expands every
cached token's per-head key and value and runs ordinary multi-head attention; section 3: it
computes the same attention as the absorbed form.
"""
import numpy as np
import torch

from mla_latent_cache_absorb_amd import workloads as wl
from oracle import latent_append as la
from oracle import mla_oracle as mo
from oracle import naive_form as nf


def bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def _tiny(rng, B=2, Q=3, L=9, H=2, D=4, R=6):
    q = bits(rng.standard_normal((B, Q, H, D)))
    cache = bits(rng.standard_normal((B, L, R)))
    w_k = bits(rng.standard_normal((H, D, R)) / 2)
    w_v = bits(rng.standard_normal((H, D, R)) / 2)
    return q, cache, w_k, w_v


def test_one_hot_latent_expands_to_a_weight_column():
    # c_j = e_r: k_{j,h} = U_h^K[:, r] and v_{j,h} = U_h^V[:, r]
    rng = np.random.default_rng(1)
    _, _, w_k, w_v = _tiny(rng)
    cache = np.zeros((6, 6), np.float32)
    cache[np.arange(6), np.arange(6)] = 1.0
    k, v = nf.expanded_kv(bits(cache), w_k, w_v, 6)
    for r in range(6):
        np.testing.assert_array_equal(k[r], mo.bf16_bits_to_f64(w_k)[:, :, r])
        np.testing.assert_array_equal(v[r], mo.bf16_bits_to_f64(w_v)[:, :, r])


def test_stages_compose_to_the_reference():
    rng = np.random.default_rng(2)
    q, cache, w_k, w_v = _tiny(rng)
    lens = np.array([9, 5])
    ref, ref_lse = mo.mla_reference(q, cache, w_k, w_v, lens, 0.5)
    for b in range(2):
        k, v = nf.expanded_kv(cache[b], w_k, w_v, int(lens[b]))
        out, lse = nf.attention_on_expanded(q[b], k, v, int(lens[b]), 0.5)
        np.testing.assert_allclose(out, ref[b], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse[b], rtol=1e-13, atol=1e-13)


def test_attention_stage_against_torch_sdpa():
    # a library routine: torch fp64 scaled_dot_product_attention with an explicit causal mask
    rng = np.random.default_rng(3)
    q, cache, w_k, w_v = _tiny(rng, B=1, Q=4, L=7)
    k, v = nf.expanded_kv(cache[0], w_k, w_v, 7)
    out, _ = nf.attention_on_expanded(q[0], k, v, 7, 0.5)
    qt = torch.from_numpy(mo.bf16_bits_to_f64(q[0])).permute(1, 0, 2)       # [H, Q, D]
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    mask = torch.tensor([[j <= 7 - 4 + i for j in range(7)] for i in range(4)])
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.5)
    np.testing.assert_allclose(out, want.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_bf16_expansion_stays_within_the_parity_bar():
    # rounding the expanded keys and values to bf16 (what a GPU naive form stores) moves the
    # output by less than half the parity bar on the workload's distributions (about a quarter)
    spec = wl.make_spec(1, 3, 64, heads=64, workload_id=701)
    w = wl.make_workload(spec)
    ref, _ = mo.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, spec.scale, heads=range(4))
    k, v = nf.expanded_kv(w.cache[0], w.w_k, w.w_v, 64)
    kr = mo.bf16_bits_to_f64(la.f64_to_bf16_bits(k))
    vr = mo.bf16_bits_to_f64(la.f64_to_bf16_bits(v))
    out, _ = nf.attention_on_expanded(w.q[0], kr, vr, 64, spec.scale, heads=range(4))
    err = np.abs(out - ref[0]).max()
    assert err <= 0.5 * (1e-2 * np.abs(ref).max() + 1e-3), err


def test_planted_off_by_one_causality_is_caught():
    rng = np.random.default_rng(4)
    q, cache, w_k, w_v = _tiny(rng, B=1, Q=3, L=8)
    k, v = nf.expanded_kv(cache[0], w_k, w_v, 8)
    good, _ = nf.attention_on_expanded(q[0], k, v, 8, 0.5)
    late, _ = nf.attention_on_expanded(q[0], k, v, 9, 0.5)   # every query one position later
    ref, _ = mo.mla_reference(q, cache, w_k, w_v, np.array([8]), 0.5)
    np.testing.assert_allclose(good, ref[0], rtol=1e-13, atol=1e-13)
    assert not np.allclose(late[:2], ref[0][:2])
